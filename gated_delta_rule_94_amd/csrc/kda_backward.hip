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
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

struct BwdParams {
  const void *q, *k, *v, *g, *beta, *dO;
  const float *h0, *dhT;
  const unsigned char* records;
  const float* states;  // start state of chunk c >= 1 of unit u at (u (nch - 1) + c - 1) DK DV
  float* dstates;       // adjoint of the state at the end of chunk c of unit u at (u nch + c) DK DV
  float* grads;         // per (chunk, head) item: GradLayout::FLOATS
  void *dq, *dk, *dv, *dg, *dbeta;
  float* dh0;
  int T, H, nch;
  int64_t items;
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

// ------------------------------------------------------------------------------------------------
// 2. adjoint chain.  One workgroup per (sequence, head, 32 value columns); the record's first four
// fields (-W, Q Gamma, Kd^T, P) are copied to LDS as stored, dO's slice and dU in fp32.
template <bool F32, int DK, int DV, int C>
struct BChainCfg {
  using R = Rec<F32, DK, DV, C>;
  using E = typename Op<F32>::E;
  static constexpr int WS = 32, NSL = DV / WS, CP = R::CP, SS = WS + 1;
  static constexpr int OFF_REC = 0;                          // E [R::UT]  (NW, QG, KPT, P)
  static constexpr int OFF_GAM = (int)(R::UT * sizeof(E));   // f32 [DK]
  static constexpr int OFF_DO = OFF_GAM + DK * 4;            // f32 [C][WS]
  static constexpr int OFF_DU = OFF_DO + C * WS * 4;         // f32 [C][WS]
  static constexpr int OFF_DS = OFF_DU + C * WS * 4;         // f32 [DK][SS]
  static constexpr int TOTAL = OFF_DS + DK * SS * 4;
  static_assert(OFF_GAM % 16 == 0, "record prefix is a whole number of 16-byte vectors");
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

template <bool F32, int DK, int DV, int C>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdParams p) {
  using Cf = BChainCfg<F32, DK, DV, C>;
  using R = typename Cf::R;
  using E = typename Cf::E;
  constexpr int WS = Cf::WS, CP = Cf::CP, SS = Cf::SS;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  const E* sR = reinterpret_cast<const E*>(smem + Cf::OFF_REC);
  float* sGam = reinterpret_cast<float*>(smem + Cf::OFF_GAM);
  float* sdO = reinterpret_cast<float*>(smem + Cf::OFF_DO);
  float* sdU = reinterpret_cast<float*>(smem + Cf::OFF_DU);
  float* sdS = reinterpret_cast<float*>(smem + Cf::OFF_DS);

  const int tid = threadIdx.x;
  const int unit = blockIdx.x / Cf::NSL, col0 = (blockIdx.x % Cf::NSL) * WS;
  const int H = p.H, b = unit / H, h = unit - b * H;
  for (int e = tid; e < DK * WS; e += 256) {
    const int c = e / WS, j = e - c * WS;
    sdS[c * SS + j] = p.dhT ? p.dhT[((int64_t)unit * DK + c) * DV + col0 + j] : 0.f;
  }
  for (int ch = p.nch - 1; ch >= 0; --ch) {
    const int nr = min(C, p.T - ch * C);
    __syncthreads();  // dS of the previous step complete; the record buffers are free
    float* ds_out = p.dstates + ((int64_t)unit * p.nch + ch) * DK * DV + col0;
    for (int e = tid; e < DK * WS; e += 256) {
      const int c = e / WS, j = e - c * WS;
      ds_out[(int64_t)c * DV + j] = sdS[c * SS + j];
    }
    const unsigned char* rec = p.records + ((int64_t)(b * p.nch + ch) * H + h) * R::BYTES;
    for (int e = tid; e < Cf::OFF_GAM / 16; e += 256)
      reinterpret_cast<uint4*>(smem)[e] = reinterpret_cast<const uint4*>(rec)[e];
    for (int e = tid; e < DK; e += 256) sGam[e] = reinterpret_cast<const float*>(rec + R::GAM_BYTE)[e];
    const int64_t orow = ((int64_t)b * p.T + (int64_t)ch * C) * H + h;
    for (int e = tid; e < C * WS; e += 256) {
      const int r = e / WS, j = e - r * WS;
      sdO[e] = r < nr ? ldg<F32>(p.dO, (orow + (int64_t)r * H) * DV + col0 + j) : 0.f;
    }
    __syncthreads();
    // dU[i][j] = sum_{r >= i} P[r][i] dO[r][j] + sum_c Kd^T[c][i] dS[c][j]
    for (int mt = tid; mt < (C / 4) * (WS / 2); mt += 256) {
      const int i0 = 4 * (mt / (WS / 2)), j0 = 2 * (mt % (WS / 2));
      float acc[4][2];
      zero(acc);
      // rows r >= i0 lie in P's written tiles; above the diagonal inside a 16-row tile P is zero
      mac(acc, i0, C, [&](int i, int r) { return tf(sR[R::P + r * CP + i0 + i]); },
          [&](int r, int j) { return sdO[r * WS + j0 + j]; });
      mac(acc, 0, DK, [&](int i, int c) { return tf(sR[R::KPT + c * CP + i0 + i]); },
          [&](int c, int j) { return sdS[c * SS + j0 + j]; });
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) sdU[(i0 + i) * WS + j0 + j] = acc[i][j];
    }
    __syncthreads();
    // dS[c][j] <- e^{gl_c} dS[c][j] + sum_r QG[r][c] dO[r][j] + sum_i (-W)[i][c] dU[i][j]
    for (int mt = tid; mt < (DK / 4) * (WS / 4); mt += 256) {
      const int c0 = 4 * (mt / (WS / 4)), j0 = 4 * (mt % (WS / 4));
      float acc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = sGam[c0 + i] * sdS[(c0 + i) * SS + j0 + j];
      mac(acc, 0, C, [&](int i, int r) { return tf(sR[R::QG + r * DK + c0 + i]); },
          [&](int r, int j) { return sdO[r * WS + j0 + j]; });
      mac(acc, 0, C, [&](int i, int r) { return tf(sR[R::NW + r * DK + c0 + i]); },
          [&](int r, int j) { return sdU[r * WS + j0 + j]; });
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sdS[(c0 + i) * SS + j0 + j] = acc[i][j];
    }
  }
  __syncthreads();
  if (p.dh0)
    for (int e = tid; e < DK * WS; e += 256) {
      const int c = e / WS, j = e - c * WS;
      p.dh0[((int64_t)unit * DK + c) * DV + col0 + j] = sdS[c * SS + j];
    }
}

// ------------------------------------------------------------------------------------------------
// 3. products with the chunk's start state S0 and end adjoint dS1, one workgroup per (chunk, head).
// S0, dS1 and dO are staged in LDS in the input type, U and dU in fp32; rows padded by 16 bytes.
template <bool F32, int DK, int DV, int C>
struct BStateCfg {
  using R = Rec<F32, DK, DV, C>;
  using E = typename Op<F32>::E;
  using GL = GradLayout<DK, DV, C>;
  static constexpr int ES = sizeof(E), SE = DV + 16 / ES, SF = DV + 4;
  static constexpr int OFF_S0 = 0;                       // E [DK][SE]
  static constexpr int OFF_DS = OFF_S0 + DK * SE * ES;   // E [DK][SE]
  static constexpr int OFF_DO = OFF_DS + DK * SE * ES;   // E [C][SE]
  static constexpr int OFF_U = OFF_DO + C * SE * ES;     // f32 [C][SF]
  static constexpr int OFF_DU = OFF_U + C * SF * 4;      // f32 [C][SF]
  static constexpr int TOTAL = OFF_DU + C * SF * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

template <bool F32, int DK, int DV, int C>
__global__ __launch_bounds__(256) void bwd_state_kernel(BwdParams p) {
  using Cf = BStateCfg<F32, DK, DV, C>;
  using R = typename Cf::R;
  using E = typename Cf::E;
  using GL = typename Cf::GL;
  constexpr int SE = Cf::SE, SF = Cf::SF, CP = R::CP;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  E* sS0 = reinterpret_cast<E*>(smem + Cf::OFF_S0);
  E* sdS = reinterpret_cast<E*>(smem + Cf::OFF_DS);
  E* sdO = reinterpret_cast<E*>(smem + Cf::OFF_DO);
  float* sU = reinterpret_cast<float*>(smem + Cf::OFF_U);
  float* sdU = reinterpret_cast<float*>(smem + Cf::OFF_DU);

  const int64_t item = blockIdx.x;
  if (item >= p.items) return;
  const int tid = threadIdx.x, H = p.H;
  const int64_t cg = item / H;
  const int h = (int)(item - cg * H), b = (int)(cg / p.nch), ch = (int)(cg - (int64_t)b * p.nch);
  const int64_t unit = (int64_t)b * H + h;
  const int nr = min(C, p.T - ch * C);
  const E* rec = reinterpret_cast<const E*>(p.records + item * R::BYTES);
  const float* gam = reinterpret_cast<const float*>(p.records + item * R::BYTES + R::GAM_BYTE);
  const float* s0 = ch > 0 ? p.states + (unit * (p.nch - 1) + ch - 1) * DK * DV
                           : (p.h0 ? p.h0 + unit * DK * DV : nullptr);  // nullptr: zero start state
  const float* ds1 = p.dstates + (unit * p.nch + ch) * DK * DV;
  float* gr = p.grads + item * GL::FLOATS;

  for (int e = tid; e < DK * DV / 4; e += 256) {
    const int c = (4 * e) / DV, j = 4 * e - c * DV;
    const float4 a = s0 ? reinterpret_cast<const float4*>(s0)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 d = reinterpret_cast<const float4*>(ds1)[e];
    E* pa = sS0 + c * SE + j;
    E* pd = sdS + c * SE + j;
    pa[0] = (E)a.x; pa[1] = (E)a.y; pa[2] = (E)a.z; pa[3] = (E)a.w;
    pd[0] = (E)d.x; pd[1] = (E)d.y; pd[2] = (E)d.z; pd[3] = (E)d.w;
  }
  const int64_t orow = ((int64_t)b * p.T + (int64_t)ch * C) * H + h;
  for (int e = tid; e < C * DV; e += 256) {
    const int r = e / DV, j = e - r * DV;
    sdO[r * SE + j] = (E)(r < nr ? ldg<F32>(p.dO, (orow + (int64_t)r * H) * DV + j) : 0.f);
  }
  __syncthreads();
  // U[r][j] = U~[r][j] + sum_c (-W)[r][c] S0[c][j];  dU[r][j] = sum_{s >= r} P[s][r] dO[s][j] + sum_c Kd^T[c][r] dS1[c][j]
  for (int mt = tid; mt < (C / 4) * (DV / 4); mt += 256) {
    const int r0 = 4 * (mt / (DV / 4)), j0 = 4 * (mt % (DV / 4));
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = tf(rec[R::UT + (j0 + j) * C + r0 + i]);
    mac(acc, 0, DK, [&](int i, int c) { return tf(rec[R::NW + (r0 + i) * DK + c]); },
        [&](int c, int j) { return tf(sS0[c * SE + j0 + j]); });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sU[(r0 + i) * SF + j0 + j] = acc[i][j];
    zero(acc);
    mac(acc, r0, C, [&](int i, int s) { return tf(rec[R::P + s * CP + r0 + i]); },
        [&](int s, int j) { return tf(sdO[s * SE + j0 + j]); });
    mac(acc, 0, DK, [&](int i, int c) { return tf(rec[R::KPT + c * CP + r0 + i]); },
        [&](int c, int j) { return tf(sdS[c * SE + j0 + j]); });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sdU[(r0 + i) * SF + j0 + j] = acc[i][j];
        gr[GL::DU + (r0 + i) * DV + j0 + j] = acc[i][j];
      }
  }
  __syncthreads();
  // dP[r][i] = sum_j dO[r][j] U[i][j] for i <= r
  for (int mt = tid; mt < (C / 4) * (C / 4); mt += 256) {
    const int r0 = 4 * (mt / (C / 4)), i0 = 4 * (mt % (C / 4));
    float acc[4][4];
    zero(acc);
    if (i0 <= r0 + 3)
      mac(acc, 0, DV, [&](int i, int j) { return tf(sdO[(r0 + i) * SE + j]); },
          [&](int j, int n) { return sU[(i0 + n) * SF + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) gr[GL::DP + (r0 + i) * C + i0 + n] = (i0 + n <= r0 + i) ? acc[i][n] : 0.f;
  }
  // d(Q Gamma) = dO S0^T, dKd = U dS1^T, dW = -dU S0^T   ([C][DK] each)
  for (int mt = tid; mt < (C / 4) * (DK / 4); mt += 256) {
    const int r0 = 4 * (mt / (DK / 4)), c0 = 4 * (mt % (DK / 4));
    float a1[4][4], a2[4][4], a3[4][4];
    zero(a1);
    zero(a2);
    zero(a3);
    for (int j = 0; j < DV; ++j) {
      float o4[4], u4[4], du4[4], s4[4], d4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o4[i] = tf(sdO[(r0 + i) * SE + j]);
        u4[i] = sU[(r0 + i) * SF + j];
        du4[i] = sdU[(r0 + i) * SF + j];
        s4[i] = tf(sS0[(c0 + i) * SE + j]);
        d4[i] = tf(sdS[(c0 + i) * SE + j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          a1[i][n] = fmaf(o4[i], s4[n], a1[i][n]);
          a2[i][n] = fmaf(u4[i], d4[n], a2[i][n]);
          a3[i][n] = fmaf(du4[i], s4[n], a3[i][n]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int o = (r0 + i) * DK + c0 + n;
        gr[GL::DQG + o] = a1[i][n];
        gr[GL::DKD + o] = a2[i][n];
        gr[GL::DW + o] = -a3[i][n];
      }
  }
  for (int c = tid; c < DK; c += 256) {
    float s = 0.f;
    for (int j = 0; j < DV; ++j) s = fmaf(tf(sS0[c * SE + j]), tf(sdS[c * SE + j]), s);
    gr[GL::DGL + c] = gam[c] * s;
  }
}

// ------------------------------------------------------------------------------------------------
// 4. through the UT transform, one 512-thread workgroup per (chunk, head).
// Ownership for [C][DK] results: thread t owns channel t % DK and rows t / DK + NRG m.
template <bool F32, int DK, int DV, int C>
struct BIntraCfg {
  using E = typename Op<F32>::E;
  static constexpr int NTH = 512, ES = sizeof(E);
  static constexpr int NRG = NTH / DK, RPT = C / NRG;            // row groups, rows per thread
  static constexpr int NRGV = NTH / DV, RPTV = C / NRGV;
  static constexpr int NCS = NTH / C, CPS = DK / NCS;            // channel slices per row (Ekk, dT)
  static constexpr int NL = (NTH / C < C) ? NTH / C : C;         // lanes per column of the inverse
  static constexpr int SK = DK + 4 / ES;                         // E row stride (one bank of skew)
  static constexpr int SG = DK + 1, SV = DV + 4 / ES, SM = C + 1;
  static constexpr int OFF_G = 0;                                // f32 [C][SG]  G, later dG
  static constexpr int OFF_Q = OFF_G + C * SG * 4;               // E [C][SK]
  static constexpr int OFF_K = OFF_Q + ((C * SK * ES + 15) & ~15);
  static constexpr int OFF_V = OFF_K + ((C * SK * ES + 15) & ~15);
  static constexpr int OFF_EKK = OFF_V + ((C * SV * ES + 15) & ~15);  // f32 [C][SM] Ekk (strict lower)
  static constexpr int OFF_L = OFF_EKK + C * SM * 4;             // f32 [C][SM] L = (I + A)^{-1}
  static constexpr int OFF_M3 = OFF_L + C * SM * 4;              // f32 [C][SM] dT -> dL -> dA -> dEkk
  static constexpr int OFF_M4 = OFF_M3 + C * SM * 4;             // f32 [C][SM] L^T dL, then dEqk
  static constexpr int OFF_BETA = OFF_M4 + C * SM * 4;           // f32 [C]
  static constexpr int OFF_DB = OFF_BETA + C * 4;                // f32 [C]
  static constexpr int OFF_RED = OFF_DB + C * 4;                 // f32 [NRG][DK]
  static constexpr int OFF_DGL = OFF_RED + NRG * DK * 4;         // f32 [DK]
  static constexpr int TOTAL = OFF_DGL + DK * 4;
  static_assert(NRG * DK == NTH && RPT * NRG == C && NCS * CPS == DK && NCS * C == NTH, "ownership");
  static_assert(NRGV * DV == NTH && RPTV * NRGV == C, "ownership");
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

template <bool F32, int DK, int DV, int C>
__global__ __launch_bounds__(512) void bwd_intra_kernel(BwdParams p) {
  using Cf = BIntraCfg<F32, DK, DV, C>;
  using E = typename Cf::E;
  using GL = GradLayout<DK, DV, C>;
  constexpr int NRG = Cf::NRG, RPT = Cf::RPT, NCS = Cf::NCS, CPS = Cf::CPS, NL = Cf::NL;
  constexpr int SK = Cf::SK, SG = Cf::SG, SV = Cf::SV, SM = Cf::SM;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];
  float* sG = reinterpret_cast<float*>(smem + Cf::OFF_G);
  E* sQ = reinterpret_cast<E*>(smem + Cf::OFF_Q);
  E* sK = reinterpret_cast<E*>(smem + Cf::OFF_K);
  E* sV = reinterpret_cast<E*>(smem + Cf::OFF_V);
  float* sEkk = reinterpret_cast<float*>(smem + Cf::OFF_EKK);
  float* sL = reinterpret_cast<float*>(smem + Cf::OFF_L);
  float* sM3 = reinterpret_cast<float*>(smem + Cf::OFF_M3);
  float* sM4 = reinterpret_cast<float*>(smem + Cf::OFF_M4);
  float* sBeta = reinterpret_cast<float*>(smem + Cf::OFF_BETA);
  float* sDb = reinterpret_cast<float*>(smem + Cf::OFF_DB);
  float* sRed = reinterpret_cast<float*>(smem + Cf::OFF_RED);
  float* sDgl = reinterpret_cast<float*>(smem + Cf::OFF_DGL);

  const int64_t item = blockIdx.x;
  if (item >= p.items) return;
  const int tid = threadIdx.x, H = p.H;
  const int64_t cg = item / H;
  const int h = (int)(item - cg * H), b = (int)(cg / p.nch), ch = (int)(cg - (int64_t)b * p.nch);
  const int nr = min(C, p.T - ch * C);
  const int64_t row0 = ((int64_t)b * p.T + (int64_t)ch * C) * H + h;  // (token, head) row of the chunk's first token
  const float* gr = p.grads + item * GL::FLOATS;

  // ---- stage q, k, v, beta (rows past the chunk's end are zero) and G = cumsum(g) per channel
  for (int e = tid; e < C * DK; e += Cf::NTH) {
    const int r = e / DK, c = e - r * DK;
    const bool ok = r < nr;
    sQ[r * SK + c] = (E)(ok ? ldg<F32>(p.q, (row0 + (int64_t)r * H) * DK + c) : 0.f);
    sK[r * SK + c] = (E)(ok ? ldg<F32>(p.k, (row0 + (int64_t)r * H) * DK + c) : 0.f);
  }
  for (int e = tid; e < C * DV; e += Cf::NTH) {
    const int r = e / DV, j = e - r * DV;
    sV[r * SV + j] = (E)(r < nr ? ldg<F32>(p.v, (row0 + (int64_t)r * H) * DV + j) : 0.f);
  }
  if (tid < C) sBeta[tid] = tid < nr ? ldg<F32>(p.beta, row0 + (int64_t)tid * H) : 0.f;
  if (tid < DK) {
    float s = 0.f;
    for (int r = 0; r < C; ++r) {
      s += r < nr ? ldg<F32>(p.g, (row0 + (int64_t)r * H) * DK + tid) : 0.f;
      sG[r * SG + tid] = s;
    }
  }
  __syncthreads();

  // ---- Ekk[r][i] = sum_c k_r[c] k_i[c] e^{G_r[c] - G_i[c]} for i < r: thread (r, channel slice),
  // slices reduced across NCS neighbouring lanes
  {
    const int r = tid / NCS, cs = tid - r * NCS;
    float kr[CPS], gr_[CPS];
#pragma unroll
    for (int m = 0; m < CPS; ++m) {
      kr[m] = tf(sK[r * SK + cs + NCS * m]);
      gr_[m] = sG[r * SG + cs + NCS * m];
    }
    for (int i = 0; i < C; ++i) {
      float s = 0.f;
      if (i < r) {
#pragma unroll
        for (int m = 0; m < CPS; ++m) {
          const int c = cs + NCS * m;
          s = fmaf(kr[m] * tf(sK[i * SK + c]), __expf(gr_[m] - sG[i * SG + c]), s);
        }
      }
#pragma unroll
      for (int o = 1; o < NCS; o <<= 1) s += __shfl_xor(s, o, NCS);
      if (cs == 0) sEkk[r * SM + i] = s;  // 0 on and above the diagonal
    }
  }
  __syncthreads();

  // ---- L = (I + A)^{-1}, A = diag(beta) Ekk: column j by forward substitution, NL lanes per column,
  // lane u holding rows u + NL m
  if (tid < C * NL) {
    const int j = tid / NL, u = tid - j * NL;
    float x[C / NL];
#pragma unroll
    for (int m = 0; m < C / NL; ++m) x[m] = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < C / NL; ++m) s = fmaf(sEkk[r * SM + u + NL * m], x[m], s);
#pragma unroll
      for (int o = 1; o < NL; o <<= 1) s += __shfl_xor(s, o, NL);
      const float val = (r == j) ? 1.f : -sBeta[r] * s;
      if (u == (r % NL)) x[r / NL] = val;
    }
#pragma unroll
    for (int m = 0; m < C / NL; ++m) sL[(u + NL * m) * SM + j] = x[m];
  }
  __syncthreads();

  // ---- dT[r][i] = sum_c dW[r][c] K[i][c] e^{G_i[c]} + sum_j dU[r][j] V[i][j] for i <= r
  {
    const int r = tid / NCS, cs = tid - r * NCS;
    constexpr int VPS = DV / NCS;
    float w[CPS], du[VPS];
#pragma unroll
    for (int m = 0; m < CPS; ++m) w[m] = gr[GL::DW + r * DK + cs + NCS * m];
#pragma unroll
    for (int m = 0; m < VPS; ++m) du[m] = gr[GL::DU + r * DV + cs + NCS * m];
    for (int i = 0; i < C; ++i) {
      float s = 0.f;
      if (i <= r) {
#pragma unroll
        for (int m = 0; m < CPS; ++m) {
          const int c = cs + NCS * m;
          s = fmaf(w[m] * tf(sK[i * SK + c]), __expf(sG[i * SG + c]), s);
        }
#pragma unroll
        for (int m = 0; m < VPS; ++m) s = fmaf(du[m], tf(sV[i * SV + cs + NCS * m]), s);
      }
#pragma unroll
      for (int o = 1; o < NCS; o <<= 1) s += __shfl_xor(s, o, NCS);
      if (cs == 0) sM3[r * SM + i] = s;
    }
  }

  // ---- owned (row, channel) accumulators; dK and dG take dKG = T^T dW now:
  // dKG[i][c] = beta_i sum_{r >= i} L[r][i] dW[r][c];  dK += dKG Gamma;  dG += dKG K Gamma
  const int oc = tid % DK, org = tid / DK;
  float aq[RPT], ak[RPT], ag[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = org + NRG * m;
    float s = 0.f;
    for (int r = i; r < C; ++r) s = fmaf(sL[r * SM + i], gr[GL::DW + r * DK + oc], s);
    s *= sBeta[i];
    const float gam = __expf(sG[i * SG + oc]);
    aq[m] = 0.f;
    ak[m] = s * gam;
    ag[m] = s * tf(sK[i * SK + oc]) * gam;
  }
  // dV[i][j] = beta_i sum_{r >= i} L[r][i] dU[r][j]
  {
    const int jv = tid % DV, rgv = tid / DV;
#pragma unroll
    for (int m = 0; m < Cf::RPTV; ++m) {
      const int i = rgv + Cf::NRGV * m;
      float s = 0.f;
      for (int r = i; r < C; ++r) s = fmaf(sL[r * SM + i], gr[GL::DU + r * DV + jv], s);
      if (i < nr) stg<F32>(p.dv, (row0 + (int64_t)i * H) * DV + jv, s * sBeta[i]);
    }
  }
  __syncthreads();

  // ---- column part of dbeta (T = L diag(beta)) and dL = dT diag(beta), column i per thread
  if (tid < C) {
    const int i = tid;
    float s = 0.f;
    for (int r = i; r < C; ++r) {
      const float t = sM3[r * SM + i];
      s = fmaf(t, sL[r * SM + i], s);
      sM3[r * SM + i] = t * sBeta[i];
    }
    sDb[i] = s;
  }
  __syncthreads();

  // ---- Y = L^T dL (into M4): Y[a][bb] = sum_{r >= max(a, bb)} L[r][a] dL[r][bb]
  for (int e = tid; e < C * C; e += Cf::NTH) {
    const int a = e / C, bb = e - a * C;
    float s = 0.f;
    for (int r = max(a, bb); r < C; ++r) s = fmaf(sL[r * SM + a], sM3[r * SM + bb], s);
    sM4[a * SM + bb] = s;
  }
  __syncthreads();
  // ---- dA = strictLower(-Y L^T) (into M3): dA[a][bb] = -sum_{s <= bb} Y[a][s] L[bb][s], a > bb
  for (int e = tid; e < C * C; e += Cf::NTH) {
    const int a = e / C, bb = e - a * C;
    float s = 0.f;
    if (a > bb)
      for (int t = 0; t <= bb; ++t) s = fmaf(sM4[a * SM + t], sL[bb * SM + t], s);
    sM3[a * SM + bb] = -s;
  }
  __syncthreads();
  // ---- row part of dbeta (A = diag(beta) Ekk), dEkk = diag(beta) dA in place; dEqk = dP into M4
  if (tid < C) {
    const int r = tid;
    float s = 0.f;
    for (int i = 0; i < r; ++i) {
      const float da = sM3[r * SM + i];
      s = fmaf(da, sEkk[r * SM + i], s);
      sM3[r * SM + i] = sBeta[r] * da;
    }
    if (r < nr) stg<F32>(p.dbeta, row0 + (int64_t)r * H, sDb[r] + s);
  }
  for (int e = tid; e < C * C; e += Cf::NTH) {
    const int r = e / C, i = e - r * C;
    sM4[r * SM + i] = gr[GL::DP + r * C + i];
  }
  __syncthreads();

  // ---- through Ekk and Eqk: for every (r, i) with i <= r and channel c, e = e^{G_r[c] - G_i[c]} <= 1
  //   row side:    dQ_r += dEqk[r][i] k_i e,  dK_r += dEkk[r][i] k_i e,  dG_r += (dEqk q_r + dEkk k_r) k_i e
  //   column side: dK_i += (dEqk[r][i] q_r + dEkk[r][i] k_r) e,  dG_i -= the same times k_i
  // (the diagonal i = r has e = 1 and no net dG)
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = org + NRG * m;
    const float Gr = sG[r * SG + oc], qr = tf(sQ[r * SK + oc]), kr = tf(sK[r * SK + oc]);
    float dq = 0.f, dk = 0.f, dg = 0.f;
    for (int i = 0; i < r; ++i) {
      const float e = __expf(Gr - sG[i * SG + oc]);
      const float ki = tf(sK[i * SK + oc]) * e;
      const float wq = sM4[r * SM + i], wk = sM3[r * SM + i];
      dq = fmaf(wq, ki, dq);
      dk = fmaf(wk, ki, dk);
      dg = fmaf(fmaf(wq, qr, wk * kr), ki, dg);
    }
    dq = fmaf(sM4[r * SM + r], kr, dq);
    dk = fmaf(sM4[r * SM + r], qr, dk);
    for (int s = r + 1; s < C; ++s) {
      const float e = __expf(sG[s * SG + oc] - Gr);
      const float u = fmaf(sM4[s * SM + r], tf(sQ[s * SK + oc]), sM3[s * SM + r] * tf(sK[s * SK + oc])) * e;
      dk += u;
      dg = fmaf(-u, kr, dg);
    }
    aq[m] += dq;
    ak[m] += dk;
    ag[m] += dg;
  }

  // ---- elementwise: Q Gamma, Kd = K e^{gl - G}, and the chunk's total decay gl
  float dglp = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = org + NRG * m;
    const float G = sG[r * SG + oc], gl = sG[(C - 1) * SG + oc];
    const float gam = __expf(G), dec = __expf(gl - G);
    const float q = tf(sQ[r * SK + oc]), k = tf(sK[r * SK + oc]);
    const float dqg = gr[GL::DQG + r * DK + oc], dkd = gr[GL::DKD + r * DK + oc];
    aq[m] = fmaf(dqg, gam, aq[m]);
    ag[m] = fmaf(dqg * q, gam, ag[m]);
    ak[m] = fmaf(dkd, dec, ak[m]);
    const float t = dkd * k * dec;
    ag[m] -= t;
    dglp += t;
  }
  sRed[org * DK + oc] = dglp;
  __syncthreads();
  if (tid < DK) {
    float s = gr[GL::DGL + tid];
    for (int o = 0; o < NRG; ++o) s += sRed[o * DK + tid];
    sDgl[tid] = s;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = org + NRG * m;
    if (r == C - 1) ag[m] += sDgl[oc];
    if (r < nr) {
      stg<F32>(p.dq, (row0 + (int64_t)r * H) * DK + oc, aq[m]);
      stg<F32>(p.dk, (row0 + (int64_t)r * H) * DK + oc, ak[m]);
    }
  }
  // ---- dg = reverse cumulative sum of dG over the chunk's rows
#pragma unroll
  for (int m = 0; m < RPT; ++m) sG[(org + NRG * m) * SG + oc] = ag[m];
  __syncthreads();
  if (tid < DK) {
    float s = 0.f;
    for (int r = C - 1; r >= 0; --r) {
      s += sG[r * SG + tid];
      if (r < nr) stg<F32>(p.dg, (row0 + (int64_t)r * H) * DK + tid, s);
    }
  }
}

// ------------------------------------------------------------------------------------------------
#define KDA_BWD_INSTANCES(X)                                                                    \
  X(false, 64, 64, 16) X(false, 64, 64, 32) X(false, 64, 64, 64)                                \
  X(false, 64, 128, 16) X(false, 64, 128, 32) X(false, 64, 128, 64)                             \
  X(false, 128, 64, 16) X(false, 128, 64, 32) X(false, 128, 64, 64)                             \
  X(false, 128, 128, 16) X(false, 128, 128, 32) X(false, 128, 128, 64)                          \
  X(true, 64, 64, 16) X(true, 64, 64, 32) X(true, 64, 64, 64)

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

// [forward workspace][states: units (nch - 1) dk dv fp32][dstates: units nch dk dv fp32]
// [grads: items GradLayout floats][o scratch: B T H dv elements], each 256-byte aligned
size_t chunked_backward_workspace(bool f32, int dk, int dv, int chunk, int B, int T, int H) {
  if (!chunked_backward_supported(f32, dk, dv, chunk)) return 0;
  const int64_t nch = (T + chunk - 1) / chunk, units = (int64_t)B * H, items = units * nch;
  size_t bytes = al256(chunked_forward_workspace(f32, dk, dv, chunk, (int64_t)B * nch, H, B, false));
  bytes += al256((size_t)(units * (nch > 0 ? nch - 1 : 0)) * dk * dv * 4);
  bytes += al256((size_t)(units * nch) * dk * dv * 4);
  bytes += al256((size_t)items * grad_floats(dk, dv, chunk) * 4);
  bytes += al256((size_t)B * T * H * dv * (f32 ? 4 : 2));
  return bytes;
}

template <bool F32, int DK, int DV, int C>
static hipError_t launch_backward_kernels(const BwdParams& p, int64_t units, void* stream) {
  static_assert(GradLayout<DK, DV, C>::FLOATS == (((int64_t)C * DV + C * C + 3 * C * DK + DK + 63) & ~(int64_t)63),
                "grad layout");
  hipLaunchKernelGGL((bwd_chain_kernel<F32, DK, DV, C>), dim3((unsigned)(units * (DV / 32))), dim3(256), 0,
                     (hipStream_t)stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.items == 0) return e;
  hipLaunchKernelGGL((bwd_state_kernel<F32, DK, DV, C>), dim3((unsigned)p.items), dim3(256), 0, (hipStream_t)stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_intra_kernel<F32, DK, DV, C>), dim3((unsigned)p.items), dim3(512), 0, (hipStream_t)stream, p);
  return hipGetLastError();
}

hipError_t launch_chunked_backward(const BackwardArgs& a) {
  if (!chunked_backward_supported(a.f32, a.dk, a.dv, a.chunk)) return hipErrorInvalidValue;
  const int C = a.chunk, nch = (a.T + C - 1) / C;
  const int64_t units = (int64_t)a.B * a.H, items = units * nch;
  if (units <= 0 || units * (a.dv / 32) > INT32_MAX || items > INT32_MAX) return hipErrorInvalidValue;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  const size_t fwd = al256(chunked_forward_workspace(a.f32, a.dk, a.dv, C, (int64_t)a.B * nch, a.H, a.B, false));
  float* states = reinterpret_cast<float*>(ws + fwd);
  const size_t st_bytes = al256((size_t)(units * (nch > 0 ? nch - 1 : 0)) * a.dk * a.dv * 4);
  float* dstates = reinterpret_cast<float*>(ws + fwd + st_bytes);
  const size_t ds_bytes = al256((size_t)(units * nch) * a.dk * a.dv * 4);
  float* grads = reinterpret_cast<float*>(ws + fwd + st_bytes + ds_bytes);
  const size_t gr_bytes = al256((size_t)items * grad_floats(a.dk, a.dv, C) * 4);
  void* o_scratch = ws + fwd + st_bytes + ds_bytes + gr_bytes;
  hipError_t e = hipSuccess;
  if (a.T > 0) {
    PrefillArgs f;
    f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.beta = a.beta;
    f.h0 = a.h0; f.o = o_scratch; f.hT = nullptr;
    f.cu_seqlens = nullptr; f.num_seqs = a.B; f.T = a.T;
    f.H = a.H; f.dk = a.dk; f.dv = a.dv; f.chunk = C; f.f32 = a.f32;
    f.workspace = ws; f.workspace_bytes = fwd; f.stream = a.stream;
    if (nch >= 2) {
      f.states = states;
      f.state_every = C;
      f.max_states = nch - 1;
    }
    if ((e = launch_chunked_forward(f)) != hipSuccess) return e;
  }
  BwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.dO = a.dO;
  p.h0 = a.h0; p.dhT = a.dhT;
  p.records = ws; p.states = states; p.dstates = dstates; p.grads = grads;
  p.dq = a.dq; p.dk = a.dk_out; p.dv = a.dv_out; p.dg = a.dg; p.dbeta = a.dbeta; p.dh0 = a.dh0;
  p.T = a.T; p.H = a.H; p.nch = nch; p.items = items;
#define KDA_BWD_LAUNCH(F, D, V, CC) \
  if (a.f32 == F && a.dk == D && a.dv == V && C == CC) return launch_backward_kernels<F, D, V, CC>(p, units, a.stream);
  KDA_BWD_INSTANCES(KDA_BWD_LAUNCH)
#undef KDA_BWD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace kda
