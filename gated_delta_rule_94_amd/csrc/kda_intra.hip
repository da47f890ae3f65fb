// KDA intra-chunk kernel on gfx950: per-chunk gate cumulative sum and the UT/WY transform.
//
// Method (Kimi K3 pages: architecture blog, "Kimi Delta Attention: the linear core" -- the
// chunkwise algorithm on specialised diagonal-plus-low-rank transitions; technical-report page,
// "Architecture at a glance" -- the scaled-sigmoid lower bound on the log-decay keeps causal
// tiles dense matrix products).  For one chunk of C tokens, G the chunk-local inclusive
// cumulative sum of the log-decay g and Gamma = e^G:
//
//   A  = diag(beta) strictLower(M_kk),   M_kk[r,i] = sum_c k_r[c] k_i[c] e^{G_r[c] - G_i[c]}
//   T  = (I + A)^{-1} diag(beta)
//   W  = T (K . Gamma),  U~ = T V,  P = lowerIncl(M_qk)  (M_qk likewise with q_r)
//
// and the chain operands Q . Gamma, (K . e^{G_last - G})^T and e^{G_last}; all go to the
// chunk's record (kda_record.h).  Every chunk of every (sequence, head) is independent, so this
// kernel is parallel over all of them; the sequential part is left to the chain kernel.
//
// Exponent safety: over a chunk G spans up to 5 C (320 at C = 64, beyond fp32), so M is
// factorised per 16-row sub-tile b against R_b = G just before the sub-tile: rows scaled by
// e^{G_r - R_b} in [e^-80, 1], columns by e^{R_b - G_i} (in [1, e^80] inside the sub-tile, <= 1
// before it).  Every factor is finite and a factor underflows only where the exact product is
// itself negligible.  All e^{..} factors come from one exp per element (the per-token decay)
// and running products inside each 16-row sub-tile.
//
// Workgroup: 8 waves, one (chunk, head) record; two workgroups share a CU (LDS <= 80 KB), so one
// workgroup's input loads overlap the other's arithmetic.  Thread (row pair rp, channel group cpl,
// sub-tile psb) owns 2 rows x 2 NQ consecutive key channels, loaded with one 8- or 16-byte access
// per row; the 8 row pairs of a sub-tile are 8 consecutive lanes, so running products over it are
// an 8-lane scan.  The contraction over the key dimension runs in NQ "quarters" of 32 channels
// each, interleaved by channel pair: quarter qt holds pair qt of every thread's group (channels
// 2 NQ cpl + 2 qt, + 1).  Which channels a quarter holds does not change the sum over all of them.
// Per quarter, pipelined so that the later quarters' loads arrive while the earlier ones compute:
//   scan       e^g and the running products (E, the sub-tile totals Tb to LDS)
//   outputs    Q.Gamma and K'^T straight to the record, (K.Gamma)^T to LDS
//   operands   every thread writes its scaled Q / K rows, K columns and gap tiles to LDS; with
//              bf16 each tile is carried as hi + lo (hi = bf16(x), lo = bf16(x - hi)) and a
//              product takes three MFMAs (hi hi + hi lo + lo hi): q.k cancels strongly, and a
//              single bf16 rounding of the scaled operands would leave P and A with errors of
//              several percent of a short sequence's output
//   products   all eight waves run the M_kk / M_qk tile-pair MFMAs (next quarter's scan beside)
// then
//   A, P       M_kk -> A (fp32, LDS), M_qk -> P (record)
//   T          16x16 diagonal blocks of (I + A)^{-1} by fp32 forward substitution; off-diagonal
//              blocks by X_ba = -L_bb sum_c A_bc X_ca on 16x16x16 MFMA in registers
//   W, U~      MFMA, straight to the record
// A and T reuse the LDS of the operand tiles; V^T is staged in the last quarter.  Products whose
// results go to memory are formed so that each lane holds four consecutive elements of a row.
// LDS rows of 8-byte fragment pieces have strides that are odd multiples of 8 bytes (72, 136),
// so the sixteen lanes of one fragment read fall on distinct banks.
//
// Optional fused steps (IntraParams): the log-decay formed from its gate pre-activation in the
// scan, g = -A sigmoid(x) (padding rows keep a decay of 1), and q, k L2-normalised per row from
// per-thread partial sums (a lane shuffle over the row pair's lanes and one LDS exchange with
// the sibling wave).
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

struct IntraParams {
  const void *q, *k, *v, *g, *beta;
  const uint8_t *qs, *ks, *vs;  // MXFP8 inputs: E8M0 scale codes of q, k, v (q, k, v hold E4M3 codes)
  const int32_t* cu;      // packed-sequence offsets [num_seqs + 1], or NULL for equal-length sequences
  const int32_t* chunk0;  // first chunk of each packed sequence [num_seqs + 1] (with cu), else NULL
  unsigned char* ws;      // records
  int num_seqs, H, T, nch;  // T: tokens per sequence (no cu) or T_total; nch: chunks per sequence (no cu)
  float gate_scale;         // > 0: g holds the gate pre-activation x, and g = -gate_scale sigmoid(x)
  int normalize_qk;         // nonzero: q and k are L2-normalised over d_k per (token, head)
};

template <bool F32, int DK, int DV, int C>
struct IntraCfg {
  using O = Op<F32>;
  using E = typename O::E;
  static constexpr int NT = C / 16;
  static constexpr int CP = Rec<F32, DK, DV, C>::CP;
  static constexpr bool SPLIT = !F32;  // bf16 operands of M carried as hi + lo parts
  static constexpr int NPART = SPLIT ? 2 : 1;
  static constexpr int QW = 32;        // channels per quarter of the key dimension
  static constexpr int NQ = DK / QW;
  static constexpr int ES = (int)sizeof(E);
  static constexpr int QS = QW + 4;    // operand-tile row stride: 72 B (bf16), 144 B (fp32)
  static constexpr int TS = CP + 4;    // [..][token] rows: 136 B for 64 bf16 tokens, 72 B for 32
  static constexpr int AS = C + 4;     // fp32 A rows
  static constexpr int NGAP = NT == 4 ? 3 : 0;  // sub-tile pairs (b, a) with b >= a + 2
  static constexpr int al(int x) { return (x + 255) & ~255; }
  static constexpr int mx(int a, int b) { return a > b ? a : b; }
  // region X during M: operand tiles of one quarter -- (Q rows, K rows scaled by e^{G - R_b};
  // K columns scaled for the diagonal sub-tile; K columns for earlier sub-tiles) x (hi, lo) -- and
  // the gap tiles (K columns pre-scaled for each pair b >= a + 2)
  static constexpr int OPB = C * QS * ES;   // one [C][QS] operand tile
  static constexpr int GPB = 16 * QS * ES;  // one gap tile
  static constexpr int OFF_GAP = 4 * NPART * OPB;
  static constexpr int M_END = OFF_GAP + NGAP * NPART * GPB;
  // region X after M: A, the diagonal inverses and T
  static constexpr int OFF_A = 0;                               // fp32 [C][AS]
  static constexpr int OFF_L = al(OFF_A + C * AS * 4);          // fp32 [NT][16][17]
  static constexpr int OFF_T = al(OFF_L + NT * 16 * 17 * 4);    // E [C][TS]
  static constexpr int X_END = OFF_T + C * TS * ES;
  // Record fields written through LDS as whole rows (16-byte accesses over full cache lines)
  // instead of 4- or 8-byte pieces straight from the registers: K'^T staged in the V^T area during
  // the quarters (V^T is written after them) where it fits; U~^T in place over the rows of V^T
  // that its own wave alone reads; -W over A and the diagonal inverses, dead once T is formed.
  static constexpr bool KPT_LDS = !F32 && DK <= DV;
  static constexpr bool UT_LDS = !F32;
  static constexpr int SW = DK + 4;  // -W rows in LDS
  static constexpr bool NW_LDS = !F32 && C * SW * ES <= OFF_T;
  // written during prep, read by the W / U~ products
  static constexpr int OFF_KGT = al(mx(M_END, X_END));          // E [DK][TS]  (K . Gamma)^T
  static constexpr int OFF_VT = al(OFF_KGT + DK * TS * ES);     // E [DV][TS]  V^T
  static constexpr int OFF_EEND = al(OFF_VT + DV * TS * ES);    // fp32 [NT][DK] e^{sub-tile total}
  static constexpr int OFF_BETA = al(OFF_EEND + NT * DK * 4);   // fp32 [C]
  static constexpr int OFF_NRM = al(OFF_BETA + C * 4);           // fp32 [NT][8][4][2] row norms (KPT_LDS)
  static constexpr int TOTAL = al(OFF_NRM + (KPT_LDS ? NT * 8 * 4 * 2 * 4 : 0));
  static_assert(TOTAL <= 163840, "LDS budget of one gfx950 workgroup");
  // minimum waves per SIMD: two 8-wave workgroups per CU (4 waves per SIMD) where their LDS fits
  static constexpr int MINW = (2 * TOTAL <= 163840) ? 4 : 2;
};

// index of sub-tile pair (b, a), b >= a + 2 (chunks of 64 only): (2,0) -> 0, (3,0) -> 1, (3,1) -> 2
__device__ __forceinline__ constexpr int gap_index(int b, int a) { return (b == 2) ? 0 : (a == 0 ? 1 : 2); }

// sub-tile pair q of the lower triangle, pairs ordered by row b then column a <= b: (0,0), (1,0),
// (1,1), (2,0), ...
__host__ __device__ constexpr int pair_row(int q) {
  int b = 0;
  while (q > b) {
    q -= b + 1;
    ++b;
  }
  return b;
}
__host__ __device__ constexpr int pair_col(int q) { return q - pair_row(q) * (pair_row(q) + 1) / 2; }

// f(integral_constant<int, I>) for I = 0 .. N-1: a loop whose index is a compile-time constant in
// the body (the tile pairs' sub-tiles and LDS offsets then fold into immediates)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// x as bf16 hi + lo (hi = bf16(x), lo = bf16(x - hi)), or x itself for fp32 operands
template <bool F32>
__device__ __forceinline__ void st2_split(void* hi, void* lo, float a, float b) {
  if constexpr (F32) {
    st2<true>(hi, a, b);
  } else {
    const uint32_t h = pack_bf16x2(a, b);
    *reinterpret_cast<uint32_t*>(hi) = h;
    const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xffff0000u);
    *reinterpret_cast<uint32_t*>(lo) = pack_bf16x2(a - ha, b - hb);
  }
}

// x of the lane D below within its 16-lane row (DPP row_shr; lanes with no source read 0), or 1
// where m = 0.  The move must run with every lane enabled -- a DPP read from a lane disabled in
// EXEC is invalid -- so the choice is arithmetic, fma(y, m, 1 - m) with m in {0, 1} (exact for
// finite y), never a select the compiler could turn into an EXEC-masked branch around the move.
template <int D>
__device__ __forceinline__ float row_shr_or1(float x, float m) {
  const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xf, 0xf, true));
  return __builtin_fmaf(y, m, 1.f - m);
}

// eight adjacent elements at an 8-byte aligned address
template <bool F32>
__device__ __forceinline__ void st8_a8(void* dst, const float (&x)[8]) {
  if constexpr (F32) {
    float2* d = reinterpret_cast<float2*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_float2(x[2 * i], x[2 * i + 1]);
  } else {
    uint2* d = reinterpret_cast<uint2*>(dst);
    d[0] = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    d[1] = make_uint2(pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
  }
}

// four adjacent elements at an 8-byte (bf16) or 16-byte (fp32) aligned address
template <bool F32>
__device__ __forceinline__ void st4(void* dst, float a, float b, float c, float d) {
  if constexpr (F32) *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
  else *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// The 2 NQ consecutive channels of one row at element offset i of a wave-uniform base (one 8- or
// 16-byte load per 16 bytes), split into channel pairs: pair qt goes to x[qt][j].  The load is
// unconditional (i must be in bounds, 2 NQ i element-aligned to the access); !ok only zeroes.
template <bool F32, int NQ>
__device__ __forceinline__ void load_group(const void* base, uint32_t i, bool ok, Raw2<F32> (&x)[NQ][2], int j) {
  static_assert(NQ == 2 || NQ == 4, "64 or 128 key channels");
  const char* b = static_cast<const char*>(base);
  if constexpr (F32) {
#pragma unroll
    for (int h = 0; h < NQ / 2; ++h) {
      const float4 w = *reinterpret_cast<const float4*>(b + 4u * i + 16u * h);
      x[2 * h][j].v = ok ? make_float2(w.x, w.y) : make_float2(0.f, 0.f);
      x[2 * h + 1][j].v = ok ? make_float2(w.z, w.w) : make_float2(0.f, 0.f);
    }
  } else if constexpr (NQ == 4) {
    const uint4 w = *reinterpret_cast<const uint4*>(b + 2u * i);
    x[0][j].w = ok ? w.x : 0u;
    x[1][j].w = ok ? w.y : 0u;
    x[2][j].w = ok ? w.z : 0u;
    x[3][j].w = ok ? w.w : 0u;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(b + 2u * i);
    x[0][j].w = ok ? w.x : 0u;
    x[1][j].w = ok ? w.y : 0u;
  }
}

// The inverse of load_group: channel pairs w (bf16) or f (fp32), pair qt at channels 2 qt, + 1 of
// a 2 NQ-channel group, stored with one 8- or 16-byte access per 16 bytes.
template <bool F32, int NQ>
__device__ __forceinline__ void store_group(void* dst, const uint32_t (&w)[NQ], const float2 (&f)[NQ]) {
  if constexpr (F32) {
#pragma unroll
    for (int h = 0; h < NQ / 2; ++h)
      reinterpret_cast<float4*>(dst)[h] = make_float4(f[2 * h].x, f[2 * h].y, f[2 * h + 1].x, f[2 * h + 1].y);
  } else if constexpr (NQ == 4) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  }
}

// ROWS rows of RB bytes each, at a stride of SB bytes in LDS (8-byte aligned), to the contiguous
// array at dst (16-byte aligned, wave-uniform), 16 bytes per access: consecutive lanes write
// consecutive 16-byte pieces, so every store covers whole cache lines.
template <int ROWS, int RB, int SB>
__device__ __forceinline__ void rows_out(const unsigned char* lds, unsigned char* dst, int tid) {
  static_assert(RB % 16 == 0 && SB % 8 == 0, "16-byte pieces of 8-byte aligned rows");
  constexpr int U = RB / 16, N = ROWS * U;
#pragma unroll
  for (int k = 0; k < (N + 511) / 512; ++k) {
    const int u = tid + 512 * k;
    if (N % 512 == 0 || u < N) {
      const int r = u / U, pc = u - r * U;
      const uint2 a = *reinterpret_cast<const uint2*>(lds + r * SB + 16 * pc);
      const uint2 b = *reinterpret_cast<const uint2*>(lds + r * SB + 16 * pc + 8);
      *reinterpret_cast<uint4*>(dst + 16u * (uint32_t)u) = make_uint4(a.x, a.y, b.x, b.y);
    }
  }
}

// OCP Microscaling (MX) inputs: a block of 32 consecutive channels shares one E8M0 scale code s,
// worth 2^(s - 127) (code 255 is NaN); each element is an FP8 E4M3 code.  gfx950 converts a pair of
// E4M3 codes and multiplies by a float scale in one instruction (checked against the E4M3
// definition on all 256 codes, subnormals and NaN included).
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return __uint_as_float(s == 0u ? 0x00400000u : (s == 255u ? 0x7fc00000u : s << 23));
}
// E4M3 codes in bytes 0-1 (hi: bytes 2-3) of w, times 2^(s - 127)
__device__ __forceinline__ float2 mx_decode2(uint32_t w, uint32_t s, bool hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const float sc = e8m0_scale(s);
  const f2_t x = hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, sc, true) : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, sc, false);
  return make_float2(x.x, x.y);
}

// (sequence start token, length) of one chunk, and the first chunk of every sequence;
// packed offsets are clamped to [0, T_total] exactly as the chunk map does.
struct ChunkPos {
  int64_t tok0;
  int len;
};

__device__ __forceinline__ void seq_range(const int32_t* cu, int s, int T, int64_t& a, int64_t& b) {
  int x = cu[s], y = cu[s + 1];
  x = x < 0 ? 0 : (x > T ? T : x);
  y = y < x ? x : (y > T ? T : y);
  a = x;
  b = y;
}

__device__ __forceinline__ ChunkPos chunk_pos(const IntraParams& p, int chunk, int C) {
  ChunkPos cp;
  int64_t a, b;
  int first;
  if (p.cu) {
    int lo = 0, hi = p.num_seqs - 1;  // last sequence whose first chunk is <= chunk
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.chunk0[mid] <= chunk) lo = mid;
      else hi = mid - 1;
    }
    seq_range(p.cu, lo, p.T, a, b);
    first = p.chunk0[lo];
  } else {
    const int s = chunk / p.nch;
    first = s * p.nch;
    a = (int64_t)s * p.T;
    b = a + p.T;
  }
  cp.tok0 = a + (int64_t)(chunk - first) * C;
  const int64_t rem = b - cp.tok0;
  cp.len = (int)(rem < C ? rem : C);
  return cp;
}

template <bool F32, int DK, int DV, int C, bool MX>
__global__ __launch_bounds__(512, (IntraCfg<F32, DK, DV, C>::MINW)) void intra_chunk_kernel(const IntraParams p) {
  static_assert(!(MX && F32), "MXFP8 inputs take the bf16 path");
  using Cf = IntraCfg<F32, DK, DV, C>;
  using O = typename Cf::O;
  using E = typename Cf::E;
  using Frag = typename O::Frag;
  using R = Rec<F32, DK, DV, C>;
  constexpr int NT = Cf::NT, CP = Cf::CP, QS = Cf::QS, TS = Cf::TS, AS = Cf::AS, QW = Cf::QW;
  constexpr bool SPLIT = Cf::SPLIT;
  constexpr int NVP = DV / 2;           // value-column pairs
  constexpr int NVU = NVP * (CP / 8);   // value units: (column pair, 8-token group)
  static_assert(128 * NT <= 512 && NVU <= 512, "one unit per thread");
  constexpr int KSQ = O::nks(QW);       // k-steps over one quarter
  constexpr int NPAIR = NT * (NT + 1) / 2;
  constexpr int NSLOT = (2 * NPAIR + 7) / 8;  // tile pairs per wave

  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  // operand tile `which` (0 Q rows, 1 K rows, 2 K diagonal columns, 3 K earlier columns), part 0 hi / 1 lo
  auto opnd = [&](int which, int part) -> E* { return reinterpret_cast<E*>(smem + (which * Cf::NPART + part) * Cf::OPB); };
  auto gapt = [&](int gi, int part) -> E* {
    return reinterpret_cast<E*>(smem + Cf::OFF_GAP + (gi * Cf::NPART + part) * Cf::GPB);
  };
  float* As = reinterpret_cast<float*>(smem + Cf::OFF_A);
  E* Ws = reinterpret_cast<E*>(smem + Cf::OFF_A);  // -W [C][SW] once T is formed (NW_LDS)
  float* Ls = reinterpret_cast<float*>(smem + Cf::OFF_L);
  E* Ts = reinterpret_cast<E*>(smem + Cf::OFF_T);
  E* KGt = reinterpret_cast<E*>(smem + Cf::OFF_KGT);
  E* Vt = reinterpret_cast<E*>(smem + Cf::OFF_VT);
  float* Eend = reinterpret_cast<float*>(smem + Cf::OFF_EEND);
  float* Bet = reinterpret_cast<float*>(smem + Cf::OFF_BETA);

  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;  // wave-uniform: per-wave work is a scalar branch
  const int H = p.H;
  // prep unit of this thread: 2 consecutive rows (a row pair of one 16-row sub-tile) x 2 NQ
  // consecutive channels, one channel pair in every quarter of the key dimension.  The 8 row pairs
  // of a sub-tile are 8 consecutive lanes, so prefix products over the sub-tile are an 8-lane
  // scan; every quarter's operands are then built by all threads.
  const int rp = tid & 7, cpl = (tid >> 3) & 15;
  const int psb = __builtin_amdgcn_readfirstlane(tid >> 7) & 3;  // sub-tile: uniform over a wave
  const bool pact = psb < NT;
  const int r0 = 16 * psb + 2 * rp;  // rows r0, r0 + 1; channels chan(qt) (+1) in quarter qt
  // value unit of this thread
  const int vcp = tid % NVP, vtg = tid / NVP;
  const bool vact = tid < NVU;

  const int total_chunks = p.cu ? p.chunk0[p.num_seqs] : p.num_seqs * p.nch;
  const int n_items = total_chunks * H;  // < 2^31: the host bounds the token count
  const int item = blockIdx.x;
  if (item >= n_items) return;  // the grid covers the bound on the number of chunks

  constexpr int NQ = Cf::NQ;
  Raw2<F32> rg[NQ][2], rq[NQ][2], rk[NQ][2], rv[8];
  // MXFP8 inputs: the E4M3 codes of this thread's q and k rows (2 NQ channels, one scale block) and
  // of its 8 v pairs, with their scale codes; decoded where they are used, so the loads stay in
  // flight until then
  uint32_t mq[2][(NQ + 1) / 2], mk[2][(NQ + 1) / 2], sq[2], sk[2], mv[8], sv[8];
  float rb;
  bool rok[2];  // rows r0, r0 + 1 lie in the chunk (the others are zero padding)
  {
    const int chunk = item / H;
    const int h = item - chunk * H;
    const ChunkPos cp = chunk_pos(p, chunk, C);
    const int64_t row0 = cp.tok0 * H + h;  // (token, head) row of the chunk's first token
    // wave-uniform bases of the chunk and 32-bit per-lane element offsets (< C H max(DK, DV))
    constexpr int EB = F32 ? 4 : 2;
    const char* gb = static_cast<const char*>(p.g) + row0 * DK * EB;
    const char* qb = static_cast<const char*>(p.q) + row0 * DK * EB;
    const char* kb = static_cast<const char*>(p.k) + row0 * DK * EB;
    const char* vb = static_cast<const char*>(p.v) + row0 * DV * EB;
    const uint32_t kstride = (uint32_t)H * DK, vstride = (uint32_t)H * DV;
    // loads are unconditional: rows past the chunk's end (len >= 1) and idle threads read a valid
    // element, then take zero
    const int last = cp.len - 1;
    rok[0] = pact && r0 <= last;
    rok[1] = pact && r0 + 1 <= last;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = pact && (r0 + j) <= last;
      const uint32_t off = (pact ? (uint32_t)(2 * NQ * cpl) : 0u) + (uint32_t)min(r0 + j, last) * kstride;
      load_group<F32, NQ>(gb, off, ok, rg, j);
      if constexpr (MX) {
        // one byte per element: element offsets are byte offsets; padding rows take code 0 (= 0)
        // with scale code 127 (= 1)
        const uint8_t* qb8 = static_cast<const uint8_t*>(p.q) + row0 * DK;
        const uint8_t* kb8 = static_cast<const uint8_t*>(p.k) + row0 * DK;
        const uint32_t soff = (uint32_t)min(r0 + j, last) * (uint32_t)(H * (DK / 32)) + (pact ? (uint32_t)(2 * NQ * cpl / 32) : 0u);
        if constexpr (NQ == 4) {
          const uint2 a = *reinterpret_cast<const uint2*>(qb8 + off), b = *reinterpret_cast<const uint2*>(kb8 + off);
          mq[j][0] = ok ? a.x : 0u;
          mq[j][1] = ok ? a.y : 0u;
          mk[j][0] = ok ? b.x : 0u;
          mk[j][1] = ok ? b.y : 0u;
        } else {
          const uint32_t a = *reinterpret_cast<const uint32_t*>(qb8 + off), b = *reinterpret_cast<const uint32_t*>(kb8 + off);
          mq[j][0] = ok ? a : 0u;
          mk[j][0] = ok ? b : 0u;
        }
        const uint32_t a = p.qs[row0 * (DK / 32) + soff], b = p.ks[row0 * (DK / 32) + soff];
        sq[j] = ok ? a : 127u;
        sk[j] = ok ? b : 127u;
      } else {
        load_group<F32, NQ>(qb, off, ok, rq, j);
        load_group<F32, NQ>(kb, off, ok, rk, j);
      }
    }
    const uint32_t vc = vact ? (uint32_t)(2 * vcp) : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool okv = vact && (8 * vtg + i) <= last;
      const uint32_t vrow = (uint32_t)min(8 * vtg + i, last);
      if constexpr (MX) {
        const uint8_t* vb8 = static_cast<const uint8_t*>(p.v) + row0 * DV;
        const uint32_t a = *reinterpret_cast<const uint16_t*>(vb8 + vc + vrow * vstride);
        const uint32_t b = p.vs[row0 * (DV / 32) + vrow * (uint32_t)(H * (DV / 32)) + vc / 32];
        mv[i] = okv ? a : 0u;
        sv[i] = okv ? b : 127u;
      } else {
        rv[i].load32(vb, vc + vrow * vstride, okv);
      }
    }
    const float bx = ldg<F32>(p.beta, row0 + (int64_t)min(tid, last) * H);
    rb = tid <= last ? bx : 0.f;
  }
  // first channel of this thread's pair in quarter qt
  auto chan = [&](int qt) -> int { return 2 * NQ * cpl + 2 * qt; };
  // this thread's q, k pair of quarter qt in row j, and its v pair of token i, as fp32
  auto qpair = [&](int qt, int j) -> float2 {
    if constexpr (MX) return mx_decode2(mq[j][qt >> 1], sq[j], (qt & 1) != 0);
    else return rq[qt][j].f();
  };
  auto kpair = [&](int qt, int j) -> float2 {
    if constexpr (MX) return mx_decode2(mk[j][qt >> 1], sk[j], (qt & 1) != 0);
    else return rk[qt][j].f();
  };
  auto vpair = [&](int i) -> float2 {
    if constexpr (MX) return mx_decode2(mv[i], sv[i], false);
    else return rv[i].f();
  };
  unsigned char* rec0 = p.ws + (int64_t)item * R::BYTES;  // wave-uniform
  float* rgam = reinterpret_cast<float*>(rec0 + R::GAM_BYTE);
  // element e of the record: the wave-uniform base plus a 32-bit per-lane offset, so that the stores
  // address from a scalar base instead of forming 64-bit lane addresses
  auto recp = [&](uint32_t e) -> E* { return reinterpret_cast<E*>(rec0 + e * (uint32_t)sizeof(E)); };

  // ---------------- per quarter of the key dimension, pipelined so that the later quarters' loads
  // arrive while the earlier ones compute:
  //   scan(0) | sync | for qt: QG/K'/KG(qt) + operands(qt) | sync | scan(qt+1) + products(qt) | sync
  // scan: E = e^{G_r - R_b} (prefix products of e^g inside the 16-row sub-tile, R_b = G before it)
  // for this thread's rows and channels, Tb = the sub-tile's total decay (to LDS as Eend); then
  // e^{R_b - G_r} = 1 / E and the suffix product e^{G_end - G_r} = Tb / E.
  const float m1 = rp >= 1 ? 1.f : 0.f, m2 = rp >= 2 ? 1.f : 0.f, m4 = rp >= 4 ? 1.f : 0.f;
  // the decay alpha = e^g of a row; with a gate pre-activation x, g = -A sigmoid(x) and padding
  // rows (x loaded as 0) keep alpha = 1
  const float gA = p.gate_scale;
  auto decay = [&](auto gate_, float x, bool ok) -> float {
    if constexpr (decltype(gate_)::value) {
      const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-x));
      return ok ? __expf(-gA * sg) : 1.f;
    } else {
      return __expf(x);
    }
  };
  auto scan_ = [&](auto gate_, int qt, float (&Ef)[2][2], float (&Tb)[2]) {
    const float2 g0 = rg[qt][0].f(), g1 = rg[qt][1].f();
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      const float a0 = decay(gate_, ch ? g0.y : g0.x, rok[0]), a1 = decay(gate_, ch ? g1.y : g1.x, rok[1]);
      float x = a0 * a1;  // this row pair's product; inclusive scan over the 8 row pairs
      x *= row_shr_or1<1>(x, m1);
      x *= row_shr_or1<2>(x, m2);
      x *= row_shr_or1<4>(x, m4);
      Ef[0][ch] = row_shr_or1<1>(x, m1) * a0;
      Ef[1][ch] = x;
      Tb[ch] = __shfl(x, (tid & 63) | 7);  // row pair 7 of this sub-tile
    }
    if (pact && rp == 7) *reinterpret_cast<float2*>(Eend + psb * DK + chan(qt)) = make_float2(Tb[0], Tb[1]);
  };
  const bool gated = gA > 0.f;  // uniform: one scan or the other, by a scalar branch
  auto scan = [&](int qt, float (&Ef)[2][2], float (&Tb)[2]) {
    if (gated) scan_(std::true_type{}, qt, Ef, Tb);
    else scan_(std::false_type{}, qt, Ef, Tb);
  };
  float Ef[2][2], Tb[2];  // this quarter's: [row j][channel]
  scan(0, Ef, Tb);
  // L2 norms of this thread's q and k rows over d_k: 8 channels here, the other 120 in the lanes
  // with the same row pair (lane bits 3-5) and in the sibling wave (through LDS, in the V^T area,
  // which is first written in the last quarter)
  float qn[2] = {1.f, 1.f}, kn[2] = {1.f, 1.f};
  // [sub-tile][row pair][4][2 halves]; in the V^T area unless K'^T is staged there
  float* Nrm = reinterpret_cast<float*>(Cf::KPT_LDS ? smem + Cf::OFF_NRM : reinterpret_cast<unsigned char*>(Vt));
  E* KPs = Vt;  // K'^T [DK][TS] during the quarters (KPT_LDS)
  const bool norm = p.normalize_qk != 0;
  if (norm) {
    float ss[4] = {0.f, 0.f, 0.f, 0.f};  // q row 0, q row 1, k row 0, k row 1
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float2 a = qpair(qt, j), b = kpair(qt, j);
        ss[j] += a.x * a.x + a.y * a.y;
        ss[2 + j] += b.x * b.x + b.y * b.y;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ss[i] += __shfl_xor(ss[i], 8);
      ss[i] += __shfl_xor(ss[i], 16);
      ss[i] += __shfl_xor(ss[i], 32);
    }
    if (pact && (lane >> 3) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Nrm[((psb * 8 + rp) * 4 + i) * 2 + (wave & 1)] = ss[i];
    }
  }
  if constexpr (CP > C) {  // token pads of K'^T and (K . Gamma)^T are zero
    for (int e = tid; e < DK * (CP - C); e += 512) {
      const int c = e / (CP - C), t = C + e % (CP - C);
      if constexpr (Cf::KPT_LDS) KPs[c * TS + t] = (E)0.f;
      else *recp(R::KPT + c * CP + t) = (E)0.f;
      KGt[c * TS + t] = (E)0.f;
    }
  }
  f32x4 acc[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) acc[sl] = zero4();
  // V^T (value unit of this thread: column pair vcp, 8 tokens from 8 vtg) to LDS
  auto write_vt = [&]() {
    if (vact) {
      float x0[8], x1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float2 vv = vpair(i);
        x0[i] = vv.x;
        x1[i] = vv.y;
      }
      st8_a8<F32>(Vt + (2 * vcp) * TS + 8 * vtg, x0);
      st8_a8<F32>(Vt + (2 * vcp + 1) * TS + 8 * vtg, x1);
    }
  };
  // Q.Gamma of this thread's rows, one channel pair per quarter, stored after the last quarter as
  // one access per row (bf16 packed pairs, or fp32 pairs)
  uint32_t qgw[2][NQ];
  float2 qgf[2][NQ];
  __syncthreads();
  if (norm && pact) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float2 a = *reinterpret_cast<const float2*>(Nrm + ((psb * 8 + rp) * 4 + j) * 2);
      const float2 b = *reinterpret_cast<const float2*>(Nrm + ((psb * 8 + rp) * 4 + 2 + j) * 2);
      qn[j] = __builtin_amdgcn_rsqf(a.x + a.y + 1e-12f);
      kn[j] = __builtin_amdgcn_rsqf(b.x + b.y + 1e-12f);
    }
  }

#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    if (pact) {
      const int c0 = chan(qt);
      // q, k as fp32 and 1 / E
      float qf[2][2], kf[2][2], iE[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float2 qq = qpair(qt, j), kk = kpair(qt, j);
        qf[j][0] = qq.x;
        qf[j][1] = qq.y;
        kf[j][0] = kk.x;
        kf[j][1] = kk.y;
        if (norm) {
          qf[j][0] *= qn[j];
          qf[j][1] *= qn[j];
          kf[j][0] *= kn[j];
          kf[j][1] *= kn[j];
        }
        iE[j][0] = __builtin_amdgcn_rcpf(Ef[j][0]);
        iE[j][1] = __builtin_amdgcn_rcpf(Ef[j][1]);
      }
      // Q.Gamma and K'^T to the record, (K.Gamma)^T to LDS: the prefix decay eP of the earlier
      // sub-tiles and the suffix decay eS of the later ones (the sub-tile is wave-uniform)
      float eP[2] = {1.f, 1.f}, eS[2] = {1.f, 1.f};
#pragma unroll
      for (int x = 0; x < NT; ++x) {
        const float2 e = *reinterpret_cast<const float2*>(Eend + x * DK + c0);
        if (x < psb) { eP[0] *= e.x; eP[1] *= e.y; }
        if (x > psb) { eS[0] *= e.x; eS[1] *= e.y; }
      }
      if (psb == 0 && rp == 0) {  // e^{G_last} = eS of sub-tile 0 times its own total
        *reinterpret_cast<float2*>(rgam + c0) = make_float2(eS[0] * Tb[0], eS[1] * Tb[1]);
      }
      {
        float qg[2][2], kg[2][2], kp[2][2];  // [row j][channel]
        const float tS[2] = {Tb[0] * eS[0], Tb[1] * eS[1]};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            const float eg = Ef[j][ch] * eP[ch];
            qg[j][ch] = qf[j][ch] * eg;
            kg[j][ch] = kf[j][ch] * eg;
            kp[j][ch] = kf[j][ch] * (iE[j][ch] * tS[ch]);
          }
          if constexpr (F32) qgf[j][qt] = make_float2(qg[j][0], qg[j][1]);
          else qgw[j][qt] = pack_bf16x2(qg[j][0], qg[j][1]);
          if (qt == NQ - 1) store_group<F32, NQ>(recp(R::QG + (r0 + j) * DK + 2 * NQ * cpl), qgw[j], qgf[j]);
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          st2<F32>(Cf::KPT_LDS ? KPs + (c0 + ch) * TS + r0 : recp(R::KPT + (c0 + ch) * CP + r0), kp[0][ch], kp[1][ch]);
          st2<F32>(KGt + (c0 + ch) * TS + r0, kg[0][ch], kg[1][ch]);
        }
      }
      // operands of this thread's rows and channels: Q and K rows scaled by E = e^{G_r - R_b}, K
      // columns for the diagonal sub-tile (1 / E = e^{R_b - G_i}), for earlier sub-tiles (Tb / E =
      // e^{G_end - G_i}) and for each gap pair (times the decay of the sub-tiles in between);
      // bf16 as hi + lo
      const int cl = 2 * cpl;
      float gp[Cf::NGAP > 0 ? Cf::NGAP : 1][2];
      if constexpr (Cf::NGAP > 0) {  // gap pairs (2,0), (3,0), (3,1): decay of the sub-tiles strictly between
        const float2 e1 = *reinterpret_cast<const float2*>(Eend + 1 * DK + c0);
        const float2 e2 = *reinterpret_cast<const float2*>(Eend + 2 * DK + c0);
        gp[0][0] = e1.x;
        gp[0][1] = e1.y;
        gp[1][0] = e1.x * e2.x;
        gp[1][1] = e1.y * e2.y;
        gp[2][0] = e2.x;
        gp[2][1] = e2.y;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = r0 + j;
        const float e0 = Ef[j][0], e1 = Ef[j][1];
        const float k0 = kf[j][0], k1 = kf[j][1];
        const float kd0 = k0 * iE[j][0], kd1 = k1 * iE[j][1];  // diagonal columns
        const float ko0 = kd0 * Tb[0], ko1 = kd1 * Tb[1];      // earlier columns
        const int o = r * QS + cl;
        st2_split<F32>(opnd(0, 0) + o, opnd(0, SPLIT) + o, qf[j][0] * e0, qf[j][1] * e1);
        st2_split<F32>(opnd(1, 0) + o, opnd(1, SPLIT) + o, k0 * e0, k1 * e1);
        st2_split<F32>(opnd(2, 0) + o, opnd(2, SPLIT) + o, kd0, kd1);
        st2_split<F32>(opnd(3, 0) + o, opnd(3, SPLIT) + o, ko0, ko1);
        if constexpr (Cf::NGAP > 0) {
          const int og = (r - 16 * psb) * QS + cl;
#pragma unroll
          for (int gi = 0; gi < Cf::NGAP; ++gi) {
            const int ga = gi == 2 ? 1 : 0;  // column sub-tile of gap pair gi
            if (psb == ga)
              st2_split<F32>(gapt(gi, 0) + og, gapt(gi, SPLIT) + og, ko0 * gp[gi][0], ko1 * gp[gi][1]);
          }
        }
      }
    }
    __syncthreads();
    // the next quarter's scan (Eend of other channels: no reader in this phase)
    if (qt + 1 < NQ) scan(qt + 1 < NQ ? qt + 1 : qt, Ef, Tb);
    // tile pairs spread over the waves; each product M^T[a-cols][b-rows] holds, per lane, row
    // r = 16 b + lo and four consecutive columns i = 16 a + 4 grp + j
    static_for<0, 2 * NPAIR>([&](auto pic) {
      constexpr int pi = decltype(pic)::value;
      if ((pi & 7) != wave) return;
      constexpr bool qk = pi >= NPAIR;
      constexpr int b = pair_row(qk ? pi - NPAIR : pi), a = pair_col(qk ? pi - NPAIR : pi);
      const int rr = (16 * b + lo) * QS;
      constexpr bool gap = b >= a + 2;
      const E* ch = gap ? gapt(gap_index(b, a), 0) + lo * QS : opnd(a == b ? 2 : 3, 0) + (16 * a + lo) * QS;
      const E* cl_ = gap ? gapt(gap_index(b, a), SPLIT) + lo * QS : opnd(a == b ? 2 : 3, SPLIT) + (16 * a + lo) * QS;
      const E* rh = opnd(qk ? 0 : 1, 0) + rr;
      const E* rl = opnd(qk ? 0 : 1, SPLIT) + rr;
      f32x4 c = acc[pi >> 3];
#pragma unroll
      for (int s = 0; s < KSQ; ++s) {
        const Frag chf = O::ld(ch, s, grp), rhf = O::ld(rh, s, grp);
        c = O::mma(chf, rhf, c);
        if constexpr (SPLIT) {
          c = O::mma(chf, O::ld(rl, s, grp), c);
          c = O::mma(O::ld(cl_, s, grp), rhf, c);
        }
      }
      acc[pi >> 3] = c;
    });
    if (qt == NQ - 1) {
      // beta and V^T (for A, T and the U~ product) last: they were loaded last; with K'^T staged
      // in the V^T area, K'^T goes to the record here and V^T follows after the barrier
      if (tid < C) Bet[tid] = rb;
      if constexpr (Cf::KPT_LDS) rows_out<DK, CP * sizeof(E), TS * sizeof(E)>(reinterpret_cast<const unsigned char*>(KPs), rec0 + R::KPT * sizeof(E), tid);
      else write_vt();
    }
    __syncthreads();
  }
  if constexpr (Cf::KPT_LDS) write_vt();  // read first by the U~ product, three barriers on

  // ---------------- M_kk -> A (fp32, LDS, strictly lower, rows scaled by beta); M_qk -> P (record)
  static_for<0, 2 * NPAIR>([&](auto pic) {
    constexpr int pi = decltype(pic)::value;
    if ((pi & 7) != wave) return;
    constexpr bool qk = pi >= NPAIR;
    constexpr int b = pair_row(qk ? pi - NPAIR : pi), a = pair_col(qk ? pi - NPAIR : pi);
    const int row = 16 * b + lo, col = 16 * a + 4 * grp;
    const f32x4 m = acc[pi >> 3];
    if constexpr (!qk) {
      const float bt = Bet[row];
      *reinterpret_cast<float4*>(As + row * AS + col) =
          make_float4(row > col ? bt * m[0] : 0.f, row > col + 1 ? bt * m[1] : 0.f, row > col + 2 ? bt * m[2] : 0.f,
                      row > col + 3 ? bt * m[3] : 0.f);
    } else {
      st4<F32>(recp(R::P + row * CP + col), row >= col ? m[0] : 0.f, row >= col + 1 ? m[1] : 0.f,
               row >= col + 2 ? m[2] : 0.f, row >= col + 3 ? m[3] : 0.f);
    }
  });
  // tiles above the diagonal that the chain's 32-deep token steps read: zero
  if constexpr (!F32) {
    for (int e = tid; e < C * 16; e += 512) {
      const int row = e >> 4, b = row >> 4;
      if ((b & 1) == 0 && 16 * (b + 1) < CP) *recp(R::P + row * CP + 16 * (b + 1) + (e & 15)) = (E)0.f;
    }
  }
  __syncthreads();

  // ---------------- diagonal 16x16 blocks of (I + A)^{-1} by forward substitution (fp32)
  if (wave < NT) {
    const int b = wave, j = lo;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* arow = As + (16 * b + r) * AS + 16 * b;
      float acc1 = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc1 -= arow[i] * x[i];
      x[r] = acc1;
    }
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Ls[(b * 16 + r) * 17 + j] = x[r];
    }
  } else if constexpr (!F32) {
    // tiles of T above the diagonal that the 32-deep token steps of W and U~ read: zero
    for (int e = tid - 64 * NT; e < C * 16; e += 512 - 64 * NT) {
      const int row = e >> 4, b = row >> 4;
      if ((b & 1) == 0 && 16 * (b + 1) < CP) Ts[row * TS + 16 * (b + 1) + (e & 15)] = (E)0.f;
    }
  }
  __syncthreads();

  // ---------------- T = (I + A)^{-1} diag(beta): column block a per wave, X_ba = -L_bb sum_c A_bc X_ca
#pragma unroll
  for (int a = 0; a < NT; ++a) {
    if (wave != a) continue;
    float Xb[NT][4];  // Xb[c][j] = X_ca[4 grp + j][lo]
    const float bcol = Bet[16 * a + lo];
#pragma unroll
    for (int j = 0; j < 4; ++j) Xb[a][j] = Ls[(a * 16 + 4 * grp + j) * 17 + lo];
#pragma unroll
    for (int r = 0; r < 4; ++r) Ts[(16 * a + 4 * grp + r) * TS + 16 * a + lo] = (E)(Xb[a][r] * bcol);
#pragma unroll
    for (int b = a + 1; b < NT; ++b) {
      f32x4 z = zero4();
#pragma unroll
      for (int c = a; c < b; ++c) {
        const float4 av4 = *reinterpret_cast<const float4*>(As + (16 * b + lo) * AS + 16 * c + 4 * grp);
        const float av[4] = {av4.x, av4.y, av4.z, av4.w};
        z = mma16<F32>(av, Xb[c], z);
      }
      float lv[4], zb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lv[j] = -Ls[(b * 16 + lo) * 17 + 4 * grp + j];
        zb[j] = z[j];
      }
      const f32x4 x = mma16<F32>(lv, zb, zero4());
#pragma unroll
      for (int j = 0; j < 4; ++j) Xb[b][j] = x[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[(16 * b + 4 * grp + r) * TS + 16 * a + lo] = (E)(x[r] * bcol);
    }
  }
  __syncthreads();

  // ---------------- -W = -T (K . Gamma) (formed transposed: 4 consecutive channels per lane) and
  // U~ = T V (U~^T: 4 consecutive tokens per lane), straight to the record
  {
    constexpr int NCT = DK / 16 + DV / 16;  // column tiles of W, then of U~
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if ((ct & 7) != wave) continue;
      const bool isw = ct < DK / 16;
      const int n16 = isw ? ct : ct - DK / 16;
      E* brow = (isw ? KGt : Vt) + (16 * n16 + lo) * TS;
      f32x4 u[NT];  // U~^T tiles, held until this wave's last read of its V^T rows
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        const E* trow = Ts + (16 * b + lo) * TS;
        f32x4 acc2 = zero4();
        if (isw) {
#pragma unroll
          for (int s = 0; s < O::nks(16 * (b + 1)); ++s) acc2 = O::mma(O::ld(brow, s, grp), O::ld(trow, s, grp), acc2);
          E* dst = Cf::NW_LDS ? Ws + (16 * b + lo) * Cf::SW + 16 * n16 + 4 * grp : recp(R::NW + (16 * b + lo) * DK + 16 * n16 + 4 * grp);
          st4<F32>(dst, -acc2[0], -acc2[1], -acc2[2], -acc2[3]);
        } else {
#pragma unroll
          for (int s = 0; s < O::nks(16 * (b + 1)); ++s) acc2 = O::mma(O::ld(trow, s, grp), O::ld(brow, s, grp), acc2);
          if constexpr (Cf::UT_LDS) u[b] = acc2;
          else st4<F32>(recp(R::UT + (16 * n16 + lo) * C + 16 * b + 4 * grp), acc2[0], acc2[1], acc2[2], acc2[3]);
        }
      }
      if (!isw && Cf::UT_LDS) {
#pragma unroll
        for (int b = 0; b < NT; ++b) st4<F32>(brow + 16 * b + 4 * grp, u[b][0], u[b][1], u[b][2], u[b][3]);
      }
    }
  }
  if constexpr (Cf::NW_LDS || Cf::UT_LDS) {
    __syncthreads();
    if constexpr (Cf::NW_LDS)
      rows_out<C, DK * sizeof(E), Cf::SW * sizeof(E)>(reinterpret_cast<const unsigned char*>(Ws), rec0 + R::NW * sizeof(E), tid);
    if constexpr (Cf::UT_LDS)
      rows_out<DV, C * sizeof(E), TS * sizeof(E)>(reinterpret_cast<const unsigned char*>(Vt), rec0 + R::UT * sizeof(E), tid);
  }
}

// Sequences that the chunk map orders by length (LDS: 4 B each).
constexpr int kOrderMax = 1024;

// Chunk map of packed sequences: chunk0[s] = sum over earlier sequences of ceil(len / C), with the
// lengths clamped to [0, T_total] as every kernel does.  One workgroup, no host synchronisation.
__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu, int num_seqs, int T, int C,
                                                        int32_t* __restrict__ chunk0, int32_t* __restrict__ order) {
  __shared__ int32_t s_part[256];
  __shared__ int32_t s_len[kOrderMax];
  const int tid = threadIdx.x;
  const int per = (num_seqs + 255) / 256;
  const int s_lo = tid * per, s_hi = min(num_seqs, s_lo + per);
  int32_t sum = 0;
  for (int s = s_lo; s < s_hi; ++s) {
    int64_t a, b;
    seq_range(cu, s, T, a, b);
    sum += (int32_t)((b - a + C - 1) / C);
  }
  s_part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive scan of the per-thread totals
    const int32_t x = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += x;
    __syncthreads();
  }
  int32_t run = s_part[tid] - sum;  // exclusive prefix
  for (int s = s_lo; s < s_hi; ++s) {
    chunk0[s] = run;
    int64_t a, b;
    seq_range(cu, s, T, a, b);
    run += (int32_t)((b - a + C - 1) / C);
  }
  if (tid == 255) chunk0[num_seqs] = s_part[255];
  // order: the sequences by decreasing chunk count (ties by index), by ranking each against all
  // others -- for up to kOrderMax sequences; beyond that, the given order
  if (num_seqs > kOrderMax) {
    for (int s = tid; s < num_seqs; s += 256) order[s] = s;
    return;
  }
  for (int s = tid; s < num_seqs; s += 256) {
    int64_t a, b;
    seq_range(cu, s, T, a, b);
    s_len[s] = (int32_t)((b - a + C - 1) / C);
  }
  __syncthreads();
  for (int s = tid; s < num_seqs; s += 256) {
    const int32_t ls = s_len[s];
    int rank = 0;
    for (int t = 0; t < num_seqs; ++t) rank += (s_len[t] > ls || (s_len[t] == ls && t < s)) ? 1 : 0;
    order[rank] = s;
  }
}

template <bool F32, int DK, int DV, int C, bool MX>
static hipError_t launch_intra_impl(const IntraLaunch& L) {
  IntraParams p;
  p.q = L.q; p.k = L.k; p.v = L.v; p.g = L.g; p.beta = L.beta;
  p.qs = L.qs; p.ks = L.ks; p.vs = L.vs;
  p.cu = L.cu; p.chunk0 = L.chunk0; p.ws = L.records;
  p.num_seqs = L.num_seqs; p.H = L.H; p.T = L.T; p.nch = L.nch;
  p.gate_scale = L.gate_scale; p.normalize_qk = L.normalize_qk ? 1 : 0;
  hipLaunchKernelGGL((intra_chunk_kernel<F32, DK, DV, C, MX>), dim3(L.grid), dim3(512), 0, (hipStream_t)L.stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_map(const int32_t* cu, int num_seqs, int T, int C, int32_t* chunk0, int32_t* order,
                            void* stream) {
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, cu, num_seqs, T, C, chunk0,
                     order);
  return hipGetLastError();
}

#define KDA_INTRA_INSTANCES(X)                                                                          \
  X(false, 64, 64, 16) X(false, 64, 64, 32) X(false, 64, 64, 64)                                        \
  X(false, 64, 128, 16) X(false, 64, 128, 32) X(false, 64, 128, 64)                                     \
  X(false, 128, 64, 16) X(false, 128, 64, 32) X(false, 128, 64, 64)                                     \
  X(false, 128, 128, 16) X(false, 128, 128, 32) X(false, 128, 128, 64)                                  \
  X(true, 64, 64, 16) X(true, 64, 64, 32) X(true, 64, 64, 64)                                           \
  X(true, 64, 128, 16) X(true, 64, 128, 32) X(true, 64, 128, 64)                                        \
  X(true, 128, 64, 16) X(true, 128, 64, 32) X(true, 128, 64, 64)                                        \
  X(true, 128, 128, 16) X(true, 128, 128, 32) X(true, 128, 128, 64)

// MXFP8 q, k, v: the bf16 shapes
#define KDA_INTRA_MX_INSTANCES(X)                                                                       \
  X(false, 64, 64, 16) X(false, 64, 64, 32) X(false, 64, 64, 64)                                        \
  X(false, 64, 128, 16) X(false, 64, 128, 32) X(false, 64, 128, 64)                                     \
  X(false, 128, 64, 16) X(false, 128, 64, 32) X(false, 128, 64, 64)                                     \
  X(false, 128, 128, 16) X(false, 128, 128, 32) X(false, 128, 128, 64)

hipError_t launch_intra(const IntraLaunch& L) {
  const bool mx = L.qs != nullptr;
#define KDA_LAUNCH(F, D, V, CC) \
  if (!mx && L.f32 == F && L.dk == D && L.dv == V && L.chunk == CC) return launch_intra_impl<F, D, V, CC, false>(L);
  KDA_INTRA_INSTANCES(KDA_LAUNCH)
#undef KDA_LAUNCH
#define KDA_LAUNCH(F, D, V, CC) \
  if (mx && L.f32 == F && L.dk == D && L.dv == V && L.chunk == CC) return launch_intra_impl<F, D, V, CC, true>(L);
  KDA_INTRA_MX_INSTANCES(KDA_LAUNCH)
#undef KDA_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kda
