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
// Workgroup: 8 waves, one (chunk, head) record.
//   prep   one thread per (2 channels, 8 rows): e^g, running products; Q.Gamma and K'^T straight
//          to the record
//   M      M_kk -> A (LDS, fp32), M_qk -> P (record): 16x16 tile pairs spread over the waves,
//          accumulated over two channel halves whose scaled operand tiles are rebuilt in LDS.
//          With bf16 operands each tile is carried as hi + lo (hi = bf16(x), lo = bf16(x - hi))
//          and a product takes three MFMAs (hi hi + hi lo + lo hi): q.k cancels strongly, and a
//          single bf16 rounding of the scaled operands would leave P and A with errors of several
//          percent of a short sequence's output
//   T      16x16 diagonal blocks of (I + A)^{-1} by fp32 forward substitution; off-diagonal
//          blocks by X_ba = -L_bb sum_c A_bc X_ca on 16x16x16 MFMA in registers
//   W, U~  MFMA, straight to the record
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

struct IntraParams {
  const void *q, *k, *v, *g, *beta;
  const int32_t* cu;      // packed-sequence offsets [num_seqs + 1], or NULL for equal-length sequences
  const int32_t* chunk0;  // first chunk of each packed sequence [num_seqs + 1] (with cu), else NULL
  unsigned char* ws;      // records
  int num_seqs, H, T, nch;  // T: tokens per sequence (no cu) or T_total; nch: chunks per sequence (no cu)
};

template <bool F32, int DK, int DV, int C>
struct IntraCfg {
  using O = Op<F32>;
  using E = typename O::E;
  static constexpr int NT = C / 16;
  static constexpr int CP = Rec<F32, DK, DV, C>::CP;
  static constexpr bool SPLIT = !F32;  // bf16 operands of M carried as hi + lo parts
  static constexpr int NPART = SPLIT ? 2 : 1;
  static constexpr int DH = DK / 2;    // channels per half: M is accumulated over two channel halves
  static constexpr int HS = DH + 8;    // stride of [token][channel-half] tiles (16-byte rows, conflict-free)
  static constexpr int TS = CP + 8;    // [..][token] tiles
  static constexpr int AS = C + 4;     // fp32 A
  static constexpr int ES = (int)sizeof(E);
  static constexpr int NGAP = NT == 4 ? 3 : 0;  // sub-tile pairs (b, a) with b >= a + 2
  static constexpr int al(int x) { return (x + 15) & ~15; }
  // R1: operands of M for one channel half -- (Q, K rows scaled by e^{G - R_b}; K columns scaled for
  // the diagonal sub-tile, for earlier sub-tiles, and pre-scaled for each gap pair) x (hi, lo) --
  // reused after M for T and the diagonal inverses
  static constexpr int OPB = C * HS * ES;      // one [C][HS] operand tile
  static constexpr int GPB = 16 * HS * ES;     // one gap tile
  static constexpr int OFF_QH = 0;
  static constexpr int OFF_KH = OFF_QH + NPART * OPB;
  static constexpr int OFF_KC = OFF_KH + NPART * OPB;
  static constexpr int OFF_KT = OFF_KC + NPART * OPB;
  static constexpr int OFF_GAP = OFF_KT + NPART * OPB;
  static constexpr int R1_END = al(OFF_GAP + NGAP * NPART * GPB);
  static constexpr int OFF_T = 0;
  static constexpr int OFF_L = al(OFF_T + C * TS * ES);
  static_assert(OFF_L + NT * 16 * 17 * 4 <= R1_END, "R1 aliases");
  static constexpr int OFF_KGT = R1_END;                    // (K . Gamma)^T  [DK][TS]
  static constexpr int OFF_VT = al(OFF_KGT + DK * TS * ES); // V^T          [DV][TS]
  static constexpr int OFF_A = al(OFF_VT + DV * TS * ES);   // A fp32       [C][AS]
  static constexpr int OFF_EEND = al(OFF_A + C * AS * 4);   // e^{sub-tile total} [NT][DK]
  static constexpr int OFF_BETA = al(OFF_EEND + NT * DK * 4);  // beta      [C]
  static constexpr int TOTAL = al(OFF_BETA + C * 4);
  static_assert(TOTAL <= 163840, "LDS budget of one gfx950 workgroup");
};

// index of sub-tile pair (b, a), b >= a + 2 (chunks of 64 only): (2,0) -> 0, (3,0) -> 1, (3,1) -> 2
__device__ __forceinline__ constexpr int gap_index(int b, int a) { return (b == 2) ? 0 : (a == 0 ? 1 : 2); }

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

template <bool F32, int DK, int DV, int C>
__global__ __launch_bounds__(512) void intra_chunk_kernel(const IntraParams p) {
  using Cf = IntraCfg<F32, DK, DV, C>;
  using O = typename Cf::O;
  using E = typename Cf::E;
  using Frag = typename O::Frag;
  using R = Rec<F32, DK, DV, C>;
  constexpr int NT = Cf::NT, CP = Cf::CP, HS = Cf::HS, TS = Cf::TS, AS = Cf::AS, DH = Cf::DH;
  constexpr bool SPLIT = Cf::SPLIT;
  constexpr int NCP = DK / 2;           // channel pairs
  constexpr int NPU = NCP * NT * 2;     // prep units: (channel pair, sub-tile, half sub-tile)
  constexpr int NVP = DV / 2;           // value-column pairs
  constexpr int NVU = NVP * (CP / 8);   // value units: (column pair, 8-token group)
  static_assert(NPU <= 512 && NVU <= 512, "one unit per thread");
  constexpr int KSH = O::nks(DH);       // k-steps over one channel half
  constexpr int NPAIR = NT * (NT + 1) / 2;
  constexpr int NSLOT = (2 * NPAIR + 7) / 8;  // tile pairs per wave

  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  // operand tile `which` (0 Q rows, 1 K rows, 2 K diagonal columns, 3 K earlier columns), part 0 hi / 1 lo
  auto opnd = [&](int which, int part) -> E* {
    return reinterpret_cast<E*>(smem + Cf::OFF_QH + (which * Cf::NPART + part) * Cf::OPB);
  };
  auto gapt = [&](int gi, int part) -> E* {
    return reinterpret_cast<E*>(smem + Cf::OFF_GAP + (gi * Cf::NPART + part) * Cf::GPB);
  };
  E* Ts = reinterpret_cast<E*>(smem + Cf::OFF_T);
  float* Ls = reinterpret_cast<float*>(smem + Cf::OFF_L);
  E* KGt = reinterpret_cast<E*>(smem + Cf::OFF_KGT);
  E* Vt = reinterpret_cast<E*>(smem + Cf::OFF_VT);
  float* As = reinterpret_cast<float*>(smem + Cf::OFF_A);
  float* Eend = reinterpret_cast<float*>(smem + Cf::OFF_EEND);
  float* Bet = reinterpret_cast<float*>(smem + Cf::OFF_BETA);

  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave work is a scalar branch
  const int H = p.H;
  // prep unit of this thread
  const int half = tid & 1, pm = tid >> 1;
  const int pcp = pm % NCP, psb = pm / NCP;
  const bool pact = tid < NPU;
  const int c0 = 2 * pcp;
  const int r0 = 16 * psb + 8 * half;
  const int chalf = c0 / DH, cl = c0 - chalf * DH;  // channel half and column inside it
  // value unit of this thread
  const int vcp = tid % NVP, vtg = tid / NVP;
  const bool vact = tid < NVU;

  const int total_chunks = p.cu ? p.chunk0[p.num_seqs] : p.num_seqs * p.nch;
  const int n_items = total_chunks * H;  // < 2^31: the host bounds the token count

  Raw2<F32> rg[8], rq[8], rk[8], rv[8];
  float rb = 0.f;
  auto load_inputs = [&](int item) {
    const int chunk = item / H;
    const int h = item - chunk * H;
    const ChunkPos cp = chunk_pos(p, chunk, C);
    const int64_t row0 = cp.tok0 * H + h;  // (token, head) row of the chunk's first token
    const int kstride = H * DK, vstride = H * DV;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = pact && (r0 + i) < cp.len;
      const int64_t off = row0 * DK + c0 + (r0 + i) * kstride;
      rg[i].load(p.g, off, ok);
      rq[i].load(p.q, off, ok);
      rk[i].load(p.k, off, ok);
      const bool okv = vact && (8 * vtg + i) < cp.len;
      rv[i].load(p.v, row0 * DV + 2 * vcp + (8 * vtg + i) * vstride, okv);
    }
    rb = (tid < cp.len) ? ldg<F32>(p.beta, row0 + tid * H) : 0.f;
  };

  {
    const int item = blockIdx.x;
    if (item >= n_items) return;  // the grid covers the bound on the number of chunks
    load_inputs(item);
    E* rec = reinterpret_cast<E*>(p.ws + (int64_t)item * R::BYTES);
    float* rgam = reinterpret_cast<float*>(p.ws + (int64_t)item * R::BYTES + R::GAM_BYTE);

    // ---------------- prep, pass 1: e^g and running products inside each 16-row sub-tile
    // E = e^{G_r - R_b} (prefix products), F = e^{G_end - G_r} (suffix products) of this thread's
    // 8 rows x 2 channels; recomputed where needed rather than kept live across the stages
    auto factors = [&](float (&E0)[8], float (&E1)[8], float (&F0)[8], float (&F1)[8]) {
      float a0[8], a1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float2 gg = rg[i].f();
        a0[i] = __expf(gg.x);
        a1[i] = __expf(gg.y);
      }
      E0[0] = a0[0];
      E1[0] = a1[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        E0[i] = E0[i - 1] * a0[i];
        E1[i] = E1[i - 1] * a1[i];
      }
      F0[7] = 1.f;
      F1[7] = 1.f;
#pragma unroll
      for (int i = 6; i >= 0; --i) {
        F0[i] = F0[i + 1] * a0[i + 1];
        F1[i] = F1[i + 1] * a1[i + 1];
      }
      // combine the two halves of the sub-tile: prefix continues from the first half, suffix from the second
      const float o0 = __shfl_xor(E0[7], 1), o1 = __shfl_xor(E1[7], 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (half) { E0[i] *= o0; E1[i] *= o1; }
        else { F0[i] *= o0; F1[i] *= o1; }
      }
    };
    {
      float E0[8], E1[8], F0[8], F1[8];
      factors(E0, E1, F0, F1);
      if (pact && half) {
        Eend[psb * DK + c0] = E0[7];
        Eend[psb * DK + c0 + 1] = E1[7];
      }
    }
    if (tid < C) Bet[tid] = rb;
    if (vact) {
      float x0[8], x1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float2 vv = rv[i].f();
        x0[i] = vv.x;
        x1[i] = vv.y;
      }
      st8<F32>(Vt + (2 * vcp) * TS + 8 * vtg, x0);
      st8<F32>(Vt + (2 * vcp + 1) * TS + 8 * vtg, x1);
    }
    __syncthreads();

    // ---------------- prep, pass 2: Q.Gamma and K'^T to the record, (K.Gamma)^T to LDS
    {
      float E0[8], E1[8], F0[8], F1[8];
      factors(E0, E1, F0, F1);
      float eP0 = 1.f, eP1 = 1.f, eS0 = 1.f, eS1 = 1.f;
#pragma unroll
      for (int x = 0; x < NT; ++x) {
        const float e0 = Eend[x * DK + c0], e1 = Eend[x * DK + c0 + 1];
        if (x < psb) { eP0 *= e0; eP1 *= e1; }
        if (x > psb) { eS0 *= e0; eS1 *= e1; }
      }
      if (pact && psb == 0 && half == 0) {
        float g0 = 1.f, g1 = 1.f;
#pragma unroll
        for (int x = 0; x < NT; ++x) { g0 *= Eend[x * DK + c0]; g1 *= Eend[x * DK + c0 + 1]; }
        *reinterpret_cast<float2*>(rgam + c0) = make_float2(g0, g1);
      }
      if (pact) {
        float kg0[8], kg1[8], kp0[8], kp1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = r0 + i;
          const float2 qq = rq[i].f(), kk = rk[i].f();
          st2<F32>(rec + R::QG + r * DK + c0, qq.x * (E0[i] * eP0), qq.y * (E1[i] * eP1));
          kg0[i] = kk.x * (E0[i] * eP0);
          kg1[i] = kk.y * (E1[i] * eP1);
          kp0[i] = kk.x * (F0[i] * eS0);
          kp1[i] = kk.y * (F1[i] * eS1);
        }
        st8<F32>(KGt + c0 * TS + r0, kg0);
        st8<F32>(KGt + (c0 + 1) * TS + r0, kg1);
        st8<F32>(rec + R::KPT + c0 * CP + r0, kp0);
        st8<F32>(rec + R::KPT + (c0 + 1) * CP + r0, kp1);
      }
    }
    if constexpr (CP > C) {  // token pad of the token-contraction operands is zero
      for (int e = tid; e < DK * (CP - C); e += 512) {
        const int c = e / (CP - C), t = C + e % (CP - C);
        KGt[c * TS + t] = (E)0.f;
        rec[R::KPT + c * CP + t] = (E)0.f;
      }
    }

    // ---------------- M_kk and M_qk over the two channel halves (operand tiles rebuilt per half)
    // operands of the threads whose channels lie in half hf: Q and K rows scaled by e^{G_r - R_b},
    // K columns for the diagonal sub-tile (e^{R_b - G_i}), for earlier sub-tiles (e^{G_end - G_i})
    // and for each gap pair (times the decay of the sub-tiles in between); bf16 as hi + lo
    auto write_operands = [&](int hf) {
      float E0[8], E1[8], F0[8], F1[8];
      factors(E0, E1, F0, F1);  // every lane: the sub-tile halves exchange partial products
      if (!pact || chalf != hf) return;
      // e^{-(sub-tile total)} turns the earlier-column factor into the diagonal one
      const float rT0 = 1.f / Eend[psb * DK + c0], rT1 = 1.f / Eend[psb * DK + c0 + 1];
      // gap pairs (2,0), (3,0), (3,1): decay of the sub-tiles strictly between
      float gp[Cf::NGAP > 0 ? Cf::NGAP : 1][2];
      if constexpr (Cf::NGAP > 0) {
        gp[0][0] = Eend[1 * DK + c0];
        gp[0][1] = Eend[1 * DK + c0 + 1];
        gp[1][0] = gp[0][0] * Eend[2 * DK + c0];
        gp[1][1] = gp[0][1] * Eend[2 * DK + c0 + 1];
        gp[2][0] = Eend[2 * DK + c0];
        gp[2][1] = Eend[2 * DK + c0 + 1];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = r0 + i;
        const float2 qq = rq[i].f(), kk = rk[i].f();
        const int o = r * HS + cl;
        st2_split<F32>(opnd(0, 0) + o, opnd(0, SPLIT) + o, qq.x * E0[i], qq.y * E1[i]);
        st2_split<F32>(opnd(1, 0) + o, opnd(1, SPLIT) + o, kk.x * E0[i], kk.y * E1[i]);
        st2_split<F32>(opnd(2, 0) + o, opnd(2, SPLIT) + o, kk.x * (F0[i] * rT0), kk.y * (F1[i] * rT1));
        st2_split<F32>(opnd(3, 0) + o, opnd(3, SPLIT) + o, kk.x * F0[i], kk.y * F1[i]);
        if constexpr (Cf::NGAP > 0) {
          const int og = (r - 16 * psb) * HS + cl;
#pragma unroll
          for (int gi = 0; gi < Cf::NGAP; ++gi) {
            const int ga = gi == 2 ? 1 : 0;  // column sub-tile of gap pair gi
            if (psb == ga)
              st2_split<F32>(gapt(gi, 0) + og, gapt(gi, SPLIT) + og, kk.x * F0[i] * gp[gi][0],
                             kk.y * F1[i] * gp[gi][1]);
          }
        }
      }
    };
    f32x4 acc[NSLOT];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) acc[sl] = zero4();
    auto accumulate = [&]() {
#pragma unroll
      for (int pi = 0; pi < 2 * NPAIR; ++pi) {
        if ((pi & 7) != wave) continue;
        const bool qk = pi >= NPAIR;
        int qq = qk ? pi - NPAIR : pi;
        int b = 0;
        while (qq > b) { qq -= b + 1; ++b; }
        const int a = qq;
        const int ar = (16 * b + lo) * HS;
        const bool gap = b >= a + 2;
        const E* bh = gap ? gapt(gap_index(b, a), 0) + lo * HS : opnd(a == b ? 2 : 3, 0) + (16 * a + lo) * HS;
        const E* bl = gap ? gapt(gap_index(b, a), SPLIT) + lo * HS : opnd(a == b ? 2 : 3, SPLIT) + (16 * a + lo) * HS;
        const E* ah = opnd(qk ? 0 : 1, 0) + ar;
        const E* al_ = opnd(qk ? 0 : 1, SPLIT) + ar;
        f32x4 c = acc[pi >> 3];
#pragma unroll
        for (int s = 0; s < KSH; ++s) {
          const Frag ahf = O::ld(ah, s, grp), bhf = O::ld(bh, s, grp);
          c = O::mma(ahf, bhf, c);
          if constexpr (SPLIT) {
            c = O::mma(ahf, O::ld(bl, s, grp), c);
            c = O::mma(O::ld(al_, s, grp), bhf, c);
          }
        }
        acc[pi >> 3] = c;
      }
    };
    write_operands(0);
    __syncthreads();
    accumulate();
    __syncthreads();
    write_operands(1);
    __syncthreads();
    accumulate();
    // M_kk -> A (fp32, LDS, strictly lower, rows scaled by beta); M_qk -> P (record, lower incl. diagonal)
#pragma unroll
    for (int pi = 0; pi < 2 * NPAIR; ++pi) {
      if ((pi & 7) != wave) continue;
      const bool qk = pi >= NPAIR;
      int qq = qk ? pi - NPAIR : pi;
      int b = 0;
      while (qq > b) { qq -= b + 1; ++b; }
      const int a = qq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * b + 4 * grp + r, col = 16 * a + lo;
        const float m = acc[pi >> 3][r];
        if (!qk) As[row * AS + col] = (row > col) ? Bet[row] * m : 0.f;
        else rec[R::P + row * CP + col] = (E)((row >= col) ? m : 0.f);
      }
    }
    // tiles above the diagonal that the chain's 32-deep token steps read: zero
    if constexpr (!F32) {
      for (int e = tid; e < C * 16; e += 512) {
        const int row = e >> 4, b = row >> 4;
        if ((b & 1) == 0 && 16 * (b + 1) < CP) rec[R::P + row * CP + 16 * (b + 1) + (e & 15)] = (E)0.f;
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
        float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc -= arow[i] * x[i];
        x[r] = acc;
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

    // ---------------- -W = -T (K . Gamma) and U~ = T V, straight to the record
    {
      constexpr int NCT = DK / 16 + DV / 16;  // column tiles of W, then of U~
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if ((ct & 7) != wave) continue;
        const bool isw = ct < DK / 16;
        const int n16 = isw ? ct : ct - DK / 16;
        const E* brow = (isw ? KGt : Vt) + (16 * n16 + lo) * TS;
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          const E* trow = Ts + (16 * b + lo) * TS;
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < O::nks(16 * (b + 1)); ++s) acc = O::mma(O::ld(trow, s, grp), O::ld(brow, s, grp), acc);
          if (isw) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[R::NW + (16 * b + 4 * grp + r) * DK + 16 * n16 + lo] = (E)(-acc[r]);
          } else {  // U~^T: this lane's 4 tokens of one column are contiguous
            E* dst = rec + R::UT + (16 * n16 + lo) * C + 16 * b + 4 * grp;
            if constexpr (F32) *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            else *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
          }
        }
      }
    }
    __syncthreads();
  }
}

// Chunk map of packed sequences: chunk0[s] = sum over earlier sequences of ceil(len / C), with the
// lengths clamped to [0, T_total] as every kernel does.  One workgroup, no host synchronisation.
__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu, int num_seqs, int T, int C,
                                                        int32_t* __restrict__ chunk0) {
  __shared__ int32_t s_part[256];
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
}

template <bool F32, int DK, int DV, int C>
static hipError_t launch_intra_impl(const IntraLaunch& L) {
  IntraParams p;
  p.q = L.q; p.k = L.k; p.v = L.v; p.g = L.g; p.beta = L.beta;
  p.cu = L.cu; p.chunk0 = L.chunk0; p.ws = L.records;
  p.num_seqs = L.num_seqs; p.H = L.H; p.T = L.T; p.nch = L.nch;
  hipLaunchKernelGGL((intra_chunk_kernel<F32, DK, DV, C>), dim3(L.grid), dim3(512), 0, (hipStream_t)L.stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_map(const int32_t* cu, int num_seqs, int T, int C, int32_t* chunk0, void* stream) {
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, cu, num_seqs, T, C, chunk0);
  return hipGetLastError();
}

#define KDA_INTRA_INSTANCES(X)                                                                          \
  X(false, 64, 64, 16) X(false, 64, 64, 32) X(false, 64, 64, 64)                                        \
  X(false, 64, 128, 16) X(false, 64, 128, 32) X(false, 64, 128, 64)                                     \
  X(false, 128, 64, 16) X(false, 128, 64, 32) X(false, 128, 64, 64)                                     \
  X(false, 128, 128, 16) X(false, 128, 128, 32) X(false, 128, 128, 64)                                  \
  X(true, 64, 64, 16) X(true, 64, 64, 32) X(true, 64, 64, 64)                                           \
  X(true, 64, 128, 16) X(true, 64, 128, 32) X(true, 64, 128, 64)                                        \
  X(true, 128, 64, 16) X(true, 128, 64, 32) X(true, 128, 128, 16) X(true, 128, 128, 32)

hipError_t launch_intra(const IntraLaunch& L) {
#define KDA_LAUNCH(F, D, V, CC) \
  if (L.f32 == F && L.dk == D && L.dv == V && L.chunk == CC) return launch_intra_impl<F, D, V, CC>(L);
  KDA_INTRA_INSTANCES(KDA_LAUNCH)
#undef KDA_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kda
