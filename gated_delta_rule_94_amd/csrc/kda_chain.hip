// KDA inter-chunk state propagation on gfx950.
//
// Sequential over the chunks of one (sequence, head), given each chunk's record (kda_record.h):
//   U  = U~ - W S            (the delta rule's writes, corrected for what S already stores)
//   O  = (Q . Gamma) S + P U
//   S  = Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
// (Kimi K3 pages: the fixed-size recurrent state, architecture blog "Why the attention stack is
// the story"; its per-channel decay and delta-rule write, "Kimi Delta Attention: the linear
// core".)  Value columns of S evolve independently (the gate acts on key rows), so each
// workgroup owns a WS-column slice of the state and the slices of one head run on different
// CUs -- exact, and it spreads even one long sequence over several CUs.
//
// Long sequences on few heads are further split into nseg segments of seg_len chunks.  The chain
// is affine in its initial state: over segment g, S_end = M_g S_start + b_g.  A summary launch runs
// segments 0..nseg-2 at once, from the zero state on the value columns (giving b_g) and from the
// identity on d_k extra columns with U~ = 0 (giving M_g); segment_combine_kernel walks the segments
// of each (sequence, head) in order, S_start(g + 1) = M_g S_start(g) + b_g in fp32; a second launch
// then runs every segment from its start state, writing o and, from the last segment, hT.
//
// Optional per call: the state after every `every` tokens of a sequence (prefix states for a
// serving cache), stored between chunk steps; and an output gate multiplying o at its stores.
//
// Workgroup: WS / 16 chain waves, each owning 16 value columns of the state, and four copy waves.
// The fp32 state lives in MFMA accumulator registers and is fed back as the B operand of the
// next chunk's products; U likewise.  The copy waves stream records from HBM into double-buffered
// LDS two chunks ahead (two register staging sets): while the chain waves compute chunk n, the
// copy waves write chunk n+1 into the other buffer and load chunk n+2.  Where two record buffers
// do not fit in LDS (fp32 records at d_k = 128, chunk 64), one buffer and one register set: the
// copy waves load chunk n+1 while the chain waves compute chunk n, then refill the buffer between
// two barriers.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

struct ChainParams {
  const unsigned char* ws;  // records, (chunk, head) order
  const float* h0;
  void* o;
  float* hT;
  const int32_t* cu;      // packed offsets, or NULL
  const int32_t* chunk0;  // first chunk per packed sequence, or NULL
  const int32_t* order;   // packed sequences by decreasing length (the order workgroups take them), or NULL
  int units, H, T, nch, dv;
  int nseg, seg_len;      // segments per (sequence, head) and their length in chunks (1, 0: whole)
  const float* sstart;    // nseg > 1: start state of every segment [units][nseg][DK][DV]
  float* send;            // summary launch: [b_g | M_g] of segments 0..nseg-2 [units][nseg-1][DK][DV+DK]
  float* states;          // or NULL: the state after every `every` tokens of a sequence,
  int every, max_states;  // [units][max_states][DK][DV]; with states_by_chunk (every = C), the state
  int states_by_chunk;    // after every full chunk at its record's slot: [(chunk) H + head][DK][DV]
  int states_bf16;        // states stored as bf16 (round to nearest even) instead of fp32
  const void* z;          // or NULL: an output gate, laid out and typed like o, multiplying o
};

template <bool F32, int DK, int DV, int C, int WS, bool ZG = false>
struct ChainCfg {
  using O = Op<F32>;
  using E = typename O::E;
  using R = Rec<F32, DK, DV, C>;
  static constexpr int NT = C / 16, CP = R::CP;
  static constexpr int NW = WS / 16;  // chain waves
  static constexpr int NH = 4;        // copy waves
  static constexpr int NTH = 64 * (NW + NH);
  static constexpr int NC = 64 * NH;  // copy threads
  static_assert(NW == 1 || NW == 2 || NW == 4, "slice of 16, 32 or 64 columns");
  static constexpr int RS = DK + 8, TS = CP + 8, US = C + 8;  // US: stride of the U~^T slice [WS][C]
  static constexpr int ES = (int)sizeof(E);
  static constexpr int EPU = 16 / ES;  // elements per 16-byte copy unit
  static constexpr int al(int x) { return (x + 15) & ~15; }
  static constexpr int B_NW = 0;
  static constexpr int B_QG = al(B_NW + C * RS * ES);
  static constexpr int B_P = al(B_QG + C * RS * ES);
  static constexpr int B_KPT = al(B_P + C * TS * ES);
  static constexpr int B_UT = al(B_KPT + DK * TS * ES);
  static constexpr int B_GAM = al(B_UT + WS * US * ES);
  // the output gate of the slice's outputs, [C][ZROW bytes] (rows padded by 16 bytes), where the
  // launch writes o (ZG) and two buffers still fit in LDS (HAS_Z; else the chain waves read it from
  // global memory at the stores)
  static constexpr int ZROW = WS * ES + 16, B_Z = al(B_GAM + DK * 4);
  static constexpr int BUF0 = B_Z, BUFZ = al(B_Z + C * ZROW);
  // record buffers in LDS: two (the copy waves fill one while the chain waves read the other), or
  // one where two do not fit (fp32 records with d_k = 128 and 64-token chunks)
  static constexpr int NBUF = 2 * BUF0 <= 163840 ? 2 : 1;
  static constexpr bool HAS_Z = ZG && NBUF * BUFZ <= 163840;
  static constexpr int BUF = HAS_Z ? BUFZ : BUF0;
  static constexpr int TOTAL = NBUF * BUF;
  static_assert(TOTAL <= 163840, "LDS budget of one gfx950 workgroup");
  // 16-byte copy units of one record slice: -W, Q.Gamma, P, K'^T, U~ slice, gamma
  static constexpr int U_NW = C * DK / EPU, U_QG = C * DK / EPU, U_P = C * CP / EPU, U_KPT = DK * CP / EPU;
  static constexpr int U_UT = WS * C / EPU, U_GAM = DK / 4;
  static constexpr int UNITS = U_NW + U_QG + U_P + U_KPT + U_UT + U_GAM;
};

// One part of a record copied by the NC copy threads in 16-byte units: NU units, UPR units per
// row.  Loads of units past the end repeat the last one (in bounds, unconditional, so the
// compiler counts outstanding loads exactly across the pipeline); their LDS stores are skipped.
// SW: bf16 tiles read as 8-byte fragment pieces are stored with the two 8-byte halves of every
// 16-byte unit swapped in rows whose bit 3 is set.  The fragment reads of 16 lanes (rows lo =
// 0..15, one piece each) then fall on distinct LDS banks; unswizzled, rows lo and lo + 8 share
// banks at these row strides.  Readers XOR their piece index with (lo >> 3) & 1.
template <int NC, int NU, int UPR, int GBASE, int GROW, int LBASE, int LROW, bool SW = false>
struct CopyPart {
  static constexpr int K = (NU + NC - 1) / NC;
  typedef uint32_t vec_t __attribute__((ext_vector_type(4 * K)));
  vec_t st;  // K 16-byte slots in one vector so that it stays in registers
  __device__ static __forceinline__ int unit(int ht, int k) {
    const int u = ht + NC * k;
    return u < NU ? u : NU - 1;
  }
  // The byte offsets of this thread's units in a record, formed once: each load addresses from the
  // wave-uniform record base (scalar registers) plus one of these 32-bit offsets, with no address
  // temporaries.  The empty asm in load() marks the offset as redefined there, so that it is not
  // hoisted out of the chunk loop as a 64-bit value, and keeps it in the same register for the
  // whole loop: no offset register is ever reused as a load destination, which would make the
  // next chunk's loads wait for every load of this one.
  struct Off {
    uint32_t o[K];
  };
  __device__ static __forceinline__ Off offsets(int ht) {
    Off f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int u = unit(ht, k);
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
      if (NU % NC != 0 && ht + NC * k >= NU) continue;  // only the last slot can be partial
      const int u = unit(ht, k);
      const int row = u / UPR;
      const uint32_t a0 = st[4 * k], a1 = st[4 * k + 1], a2 = st[4 * k + 2], a3 = st[4 * k + 3];
      uint4 v;
      if constexpr (SW) {
        const bool sw = (row >> 3) & 1;
        v.x = sw ? a2 : a0;
        v.y = sw ? a3 : a1;
        v.z = sw ? a0 : a2;
        v.w = sw ? a1 : a3;
      } else {
        v = make_uint4(a0, a1, a2, a3);
      }
      *reinterpret_cast<uint4*>(buf + LBASE + row * LROW + 16 * (u % UPR)) = v;
    }
  }
};

template <bool F32, int DK, int DV, int C, int WS, bool SUM>
__global__ __launch_bounds__(64 * (WS / 16 + 4)) void chain_kernel(const ChainParams p) {
  using Cf = ChainCfg<F32, DK, DV, C, WS, !SUM>;
  using O = typename Cf::O;
  using E = typename Cf::E;
  using R = typename Cf::R;
  using Frag = typename O::Frag;
  constexpr int NT = Cf::NT, CP = Cf::CP, RS = Cf::RS, TS = Cf::TS, US = Cf::US, EPU = Cf::EPU;
  constexpr int KSD = O::nks(DK), KSC = O::nks(CP);
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];

  // ---- (unit, segment, slice); the slices of one (unit, segment) share an XCD (block id mod 8).
  // A summary launch has DK more columns (the identity block) and no last segment.
  constexpr int NCOL = SUM ? DV + DK : DV;
  constexpr int nsl_c = NCOL / WS;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int segs = SUM ? p.nseg - 1 : p.nseg;
  const int su = (idx / nsl_c) * 8 + xcd;
  const int slice = idx - (idx / nsl_c) * nsl_c;
  if (su >= p.units * segs) return;
  const int H = p.H;
  // (sequence, head) of this workgroup: packed sequences are taken longest first, so that the
  // long chains start in the first wave of workgroups and the short ones fill in behind them
  const int ui = su / segs, seg = su - ui * segs;
  const int n = p.order ? p.order[ui / H] : ui / H, h = ui - (ui / H) * H;
  const int unit = n * H + h;
  int64_t t_begin, t_end, first, seq0;
  if (p.nseg > 1) {  // equal-length sequences
    const int64_t s0 = (int64_t)n * p.T, s1 = s0 + p.T;
    seq0 = s0;
    t_begin = s0 + (int64_t)seg * p.seg_len * C;
    t_end = t_begin + (int64_t)p.seg_len * C < s1 ? t_begin + (int64_t)p.seg_len * C : s1;
    first = (int64_t)n * p.nch + (int64_t)seg * p.seg_len;
  } else if (p.cu) {
    int x = p.cu[n], y = p.cu[n + 1];
    x = x < 0 ? 0 : (x > p.T ? p.T : x);
    y = y < x ? x : (y > p.T ? p.T : y);
    t_begin = seq0 = x;
    t_end = y;
    first = p.chunk0[n];
  } else {
    t_begin = seq0 = (int64_t)n * p.T;
    t_end = t_begin + p.T;
    first = (int64_t)n * p.nch;
  }
  const int nchunks = (int)((t_end - t_begin + C - 1) / C);
  const int col0 = slice * WS;
  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gsw = F32 ? grp : (grp ^ ((lo >> 3) & 1));  // fragment piece of this lane in swizzled bf16 tiles
  const bool chain = wave < Cf::NW;
  const int ccol = col0 + 16 * (chain ? wave : 0) + lo;  // value column of this lane
  const bool idsl = SUM && col0 >= DV;  // identity-column slice (U~ = 0)

  // ---- state S in accumulator layout: Sacc[m][r] = S[16 m + 4 grp + r][ccol]; set and used on the
  // chain waves' path only, so it is not live across the copy waves' loop
  f32x4 Sacc[DK / 16];

  // ---- record streaming: 16-byte units, global -> registers -> LDS.  Two register staging sets
  // alternate, so a record's loads are issued two chunks before it is computed.
  auto rec_of = [&](int c) -> const unsigned char* { return p.ws + ((first + c) * H + h) * R::BYTES; };
  constexpr int ES_ = Cf::ES;
  struct Stage {
    CopyPart<Cf::NC, Cf::U_NW, DK / EPU, (int)(R::NW * ES_), DK * ES_, Cf::B_NW, RS * ES_, !F32> nw;
    CopyPart<Cf::NC, Cf::U_QG, DK / EPU, (int)(R::QG * ES_), DK * ES_, Cf::B_QG, RS * ES_, !F32> qg;
    CopyPart<Cf::NC, Cf::U_P, CP / EPU, (int)(R::P * ES_), CP * ES_, Cf::B_P, TS * ES_, !F32> pp;
    CopyPart<Cf::NC, Cf::U_KPT, CP / EPU, (int)(R::KPT * ES_), CP * ES_, Cf::B_KPT, TS * ES_, !F32> kpt;
    CopyPart<Cf::NC, Cf::U_UT, C / EPU, (int)(R::UT * ES_), C * ES_, Cf::B_UT, US * ES_, !F32> ut;  // record pointer + col0 rows
    CopyPart<Cf::NC, Cf::U_GAM, Cf::U_GAM, (int)R::GAM_BYTE, 0, Cf::B_GAM, 0> gam;
    uint4 zg;  // output gate: one 16-byte unit of the chunk's [C][WS] slice per copy thread
    struct Offs {
      typename decltype(nw)::Off nw;
      typename decltype(qg)::Off qg;
      typename decltype(pp)::Off pp;
      typename decltype(kpt)::Off kpt;
      typename decltype(ut)::Off ut;
      typename decltype(gam)::Off gam;
    };
    __device__ static __forceinline__ Offs offsets(int ht) {
      return Offs{decltype(nw)::offsets(ht), decltype(qg)::offsets(ht), decltype(pp)::offsets(ht),
                  decltype(kpt)::offsets(ht), decltype(ut)::offsets(ht), decltype(gam)::offsets(ht)};
    }
    __device__ __forceinline__ void load(const unsigned char* rp, Offs& f, int col0b) {
      nw.load(rp, f.nw); kpt.load(rp, f.kpt); ut.load(rp + col0b, f.ut); gam.load(rp, f.gam);
      if constexpr (!SUM) { qg.load(rp, f.qg); pp.load(rp, f.pp); }  // a summary writes no o
    }
    __device__ __forceinline__ void store(unsigned char* b, int ht) const {
      nw.store(b, ht); kpt.store(b, ht); ut.store(b, ht); gam.store(b, ht);
      if constexpr (!SUM) { qg.store(b, ht); pp.store(b, ht); }
    }
  };
  const int ht = tid - 64 * Cf::NW;  // copy-thread index (copy waves only)
  const int ostride = H * DV;                               // output elements between consecutive tokens
  const int ocol = col0 + 16 * (chain ? wave : 0) + 4 * grp;  // first of this lane's 4 output columns
  const int col0b = (idsl ? 0 : col0) * C * ES_;  // first U~^T row of the slice
  // the output gate's units: ZU per row of the slice, C rows; rows past the chunk re-read its last
  // token (in bounds, never stored to o)
  constexpr int ZU = WS * ES_ / 16;
  static_assert(!Cf::HAS_Z || C * ZU <= Cf::NC, "one output-gate unit per copy thread");
  auto load_z = [&](Stage& st, int c) {
    const int u = ht < C * ZU ? ht : C * ZU - 1, row = u / ZU;
    const int64_t t0 = t_begin + (int64_t)c * C;
    const int len = (int)((t_end - t0) < C ? (t_end - t0) : C);
    const int64_t zi = ((t0 + (row < len ? row : len - 1)) * H + h) * DV + col0 + (u % ZU) * (16 / ES_);
    // without an output gate the unit is read from the record buffer and never stored: the copy
    // waves then issue the same loads on every call, so the compiler counts the loads in flight
    // exactly across the pipeline (a load under a runtime branch makes it wait for all of them)
    const void* zp = p.z != nullptr ? static_cast<const void*>(static_cast<const E*>(p.z) + zi) : static_cast<const void*>(p.ws);
    st.zg = *reinterpret_cast<const uint4*>(zp);
  };
  auto store_z = [&](const Stage& st, unsigned char* b) {
    if (ht < C * ZU) *reinterpret_cast<uint4*>(b + Cf::B_Z + (ht / ZU) * Cf::ZROW + 16 * (ht % ZU)) = st.zg;
  };

  // output gate: the copy waves stream each chunk's [C][WS] slice into the chunk's LDS buffer with
  // its record, and the chain waves read it there at the stores
  const bool gz = !SUM && p.z != nullptr;

  // one chunk of the chain from LDS buffer `buf`
  auto chunk_step = [&](int c, int buf) {
    const unsigned char* b = smem + buf * Cf::BUF;
    const E* Wn = reinterpret_cast<const E*>(b + Cf::B_NW);
    const E* QG = reinterpret_cast<const E*>(b + Cf::B_QG);
    const E* Ps = reinterpret_cast<const E*>(b + Cf::B_P);
    const E* Kpt = reinterpret_cast<const E*>(b + Cf::B_KPT);
    const E* Ut = reinterpret_cast<const E*>(b + Cf::B_UT);
    const float* Gam = reinterpret_cast<const float*>(b + Cf::B_GAM);
    const int64_t t0 = t_begin + (int64_t)c * C;
    const int len = (int)((t_end - t0) < C ? (t_end - t0) : C);
    const int64_t obase = (t0 * H + h) * DV;  // output element of (token t0, head h, column 0): uniform
    if (!chain) return;
    // Phases, each issuing the LDS fragment loads of the next so that LDS latency hides behind
    // MFMAs; the state update (the chunk-to-chunk critical path) comes first:
    //   1  -W fragments, U~                   2  U = U~ - W S            | K'^T fragments, gamma
    //   3  S = gamma S + K'^T U               | Q.Gamma fragments
    //   4  O^T = S_old^T (Q.Gamma)^T          | P fragments           5  O^T += U^T P^T; store
    // O is formed transposed (the state and U fragments serve as A operands unchanged), so each
    // lane holds four consecutive value columns of one token: one 8-byte store per 16 tokens.
    Frag Sf[KSD];
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk) Sf[sk] = O::from_acc(Sacc, sk);
    Frag wf[NT][KSD];
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk)
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) wf[bt][sk] = O::ld(Wn + (16 * bt + lo) * RS, sk, gsw);
    f32x4 U[NT];
    const E* ut = Ut + (16 * wave + lo) * US + 4 * gsw;  // U~^T: this lane's 4 tokens are contiguous
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      if (idsl) {
        U[bt] = zero4();
      } else if constexpr (F32) {
        const float4 x = *reinterpret_cast<const float4*>(ut + 16 * bt);
        U[bt] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        const bf16x4 x = *reinterpret_cast<const bf16x4*>(ut + 16 * bt);
        U[bt] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    Frag kf[DK / 16][KSC];
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk)
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) U[bt] = O::mma(wf[bt][sk], Sf[sk], U[bt]);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m)
#pragma unroll
      for (int sk = 0; sk < KSC; ++sk) kf[m][sk] = O::ld(Kpt + (16 * m + lo) * TS, sk, gsw);
    if constexpr (!F32) {
#pragma unroll
      for (int i = 0; i < NT * KSD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    Frag uf[KSC];
#pragma unroll
    for (int sk = 0; sk < KSC; ++sk) uf[sk] = O::from_acc(U, sk);
    Frag qf[NT][KSD];
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
      const float4 gm = *reinterpret_cast<const float4*>(Gam + 16 * m + 4 * grp);
      Sacc[m][0] *= gm.x;
      Sacc[m][1] *= gm.y;
      Sacc[m][2] *= gm.z;
      Sacc[m][3] *= gm.w;
#pragma unroll
      for (int sk = 0; sk < KSC; ++sk) Sacc[m] = O::mma(kf[m][sk], uf[sk], Sacc[m]);
    }
    if constexpr (SUM) return;
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk)
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) qf[bt][sk] = O::ld(QG + (16 * bt + lo) * RS, sk, gsw);
    __builtin_amdgcn_sched_barrier(0);

    f32x4 Ot[NT];
    Frag pf[NT][KSC];
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) Ot[bt] = zero4();
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk)
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) Ot[bt] = O::mma(Sf[sk], qf[bt][sk], Ot[bt]);
#pragma unroll
    for (int bt = 0; bt < NT; ++bt)
#pragma unroll
      for (int sk = 0; sk < O::nks(16 * (bt + 1)); ++sk) pf[bt][sk] = O::ld(Ps + (16 * bt + lo) * TS, sk, gsw);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
      for (int sk = 0; sk < O::nks(16 * (bt + 1)); ++sk) Ot[bt] = O::mma(uf[sk], pf[bt][sk], Ot[bt]);
      if (gz) {
        float zf[4];
        const int zrow = 16 * bt + lo < len ? 16 * bt + lo : len - 1;
        const unsigned char* zr =
            Cf::HAS_Z ? b + Cf::B_Z + (16 * bt + lo) * Cf::ZROW + (ocol - col0) * ES_
                      : reinterpret_cast<const unsigned char*>(static_cast<const E*>(p.z) + obase + (int64_t)zrow * ostride + ocol);
        if constexpr (F32) {
          const float4 zv = *reinterpret_cast<const float4*>(zr);
          zf[0] = zv.x; zf[1] = zv.y; zf[2] = zv.z; zf[3] = zv.w;
        } else {
          const uint2 zv = *reinterpret_cast<const uint2*>(zr);
          zf[0] = __uint_as_float(zv.x << 16); zf[1] = __uint_as_float(zv.x & 0xffff0000u);
          zf[2] = __uint_as_float(zv.y << 16); zf[3] = __uint_as_float(zv.y & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Ot[bt][i] *= zf[i];
      }
      if (16 * bt + lo < len) {
        const int64_t oi = obase + (int64_t)(16 * bt + lo) * ostride + ocol;
        if constexpr (F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.o) + oi) = make_float4(Ot[bt][0], Ot[bt][1], Ot[bt][2], Ot[bt][3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<__bf16*>(p.o) + oi) =
              make_uint2(pack_bf16x2(Ot[bt][0], Ot[bt][1]), pack_bf16x2(Ot[bt][2], Ot[bt][3]));
        }
      }
    }
  };
  // state snapshot after chunk c when it ends `every` tokens into the sequence (every is a multiple
  // of C, so only a full chunk can): the prefix states a serving cache resumes from.  Wave-uniform.
  const int rel0 = (int)(t_begin - seq0);  // tokens of the sequence before this range (a multiple of C)
  auto snapshot = [&](int c) {
    const int rel_end = rel0 + (c + 1) * C;
    if (!p.states || rel_end % p.every != 0 || t_begin + (int64_t)(c + 1) * C > t_end) return;
    const int j = rel_end / p.every - 1;
    if (!p.states_by_chunk && j >= p.max_states) return;
    const int64_t slot = p.states_by_chunk ? (first + c) * H + h : (int64_t)unit * p.max_states + j;
    // a wave-uniform base and 32-bit lane offsets derived here from an opaque zero, so that the
    // compiler keeps no store addresses live across the chunk loop
    uint32_t z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const uint32_t lane_el = (4u * grp + z) * DV + ccol;  // element offset of this lane's first value
    if (p.states_bf16) {
      char* st = reinterpret_cast<char*>(p.states) + slot * DK * DV * 2;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<__bf16*>(st + 2u * (lane_el + (uint32_t)(16 * m + r) * DV)) = (__bf16)Sacc[m][r];
    } else {
      char* st = reinterpret_cast<char*>(p.states + slot * DK * DV);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) *reinterpret_cast<float*>(st + 4u * (lane_el + (uint32_t)(16 * m + r) * DV)) = Sacc[m][r];
    }
  };

  // Chain waves compute; copy waves stream records.  The two roles run separate loops with the same
  // barriers, so each role's registers are live on its own path only.  Prologue: chunk 0 in buffer
  // 0, chunk 1 loading into s1.  Chunk indices past the last are clamped to it: those copies repeat
  // the last record into a buffer nobody reads.
  // Invariant at chunk c: buffer c&1 holds chunk c, stage (c+1)&1 holds chunk c+1, stage c&1 is
  // free; the copy waves fill buffer (c+1)&1 while the chain waves read buffer c&1.
  const int last = nchunks - 1;
  constexpr bool ONEBUF = Cf::NBUF == 1;
  if (chain) {
    if constexpr (SUM) {  // zero on the value columns, the identity on the extra ones
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[m][r] = (idsl && 16 * m + 4 * grp + r == ccol - DV) ? 1.f : 0.f;
    } else {
      const float* s0 = p.nseg > 1 ? p.sstart + ((int64_t)unit * p.nseg + seg) * DK * DV
                                   : (p.h0 ? p.h0 + (int64_t)unit * DK * DV : nullptr);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[m][r] = s0 ? s0[(16 * m + 4 * grp + r) * DV + ccol] : 0.f;
    }
    __syncthreads();
    if constexpr (ONEBUF) {
      for (int c = 0; c < nchunks; ++c) {
        chunk_step(c, 0);
        if constexpr (!SUM) snapshot(c);
        __syncthreads();  // the buffer is free
        if (c + 1 >= nchunks) break;
        __syncthreads();  // the buffer holds chunk c + 1
      }
    } else {
      for (int c = 0; c < nchunks; c += 2) {
        chunk_step(c, 0);
        if constexpr (!SUM) snapshot(c);
        __syncthreads();
        if (c + 1 >= nchunks) break;
        chunk_step(c + 1, 1);
        if constexpr (!SUM) snapshot(c + 1);
        __syncthreads();
      }
    }
    if constexpr (SUM) {
      float* se = p.send + ((int64_t)unit * (p.nseg - 1) + seg) * DK * (DV + DK);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) se[(16 * m + 4 * grp + r) * (DV + DK) + ccol] = Sacc[m][r];
    } else if (p.hT && seg == p.nseg - 1) {
      float* ht_ = p.hT + (int64_t)unit * DK * DV;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) ht_[(16 * m + 4 * grp + r) * DV + ccol] = Sacc[m][r];
    }
  } else if constexpr (ONEBUF) {
    // one buffer: chunk c + 1 waits in registers while the chain waves compute chunk c
    Stage s0;
    typename Stage::Offs offs = Stage::offsets(ht);
    if (nchunks > 0) {
      s0.load(rec_of(0), offs, col0b);
      if (Cf::HAS_Z) load_z(s0, 0);
      s0.store(smem, ht);
      if (Cf::HAS_Z && gz) store_z(s0, smem);
      s0.load(rec_of(last < 1 ? last : 1), offs, col0b);
      if (Cf::HAS_Z) load_z(s0, last < 1 ? last : 1);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      __syncthreads();  // the chain waves are done with chunk c
      if (c + 1 >= nchunks) break;
      s0.store(smem, ht);
      if (Cf::HAS_Z && gz) store_z(s0, smem);
      __syncthreads();  // the buffer holds chunk c + 1
      s0.load(rec_of(c + 2 < last ? c + 2 : last), offs, col0b);
      if (Cf::HAS_Z) load_z(s0, c + 2 < last ? c + 2 : last);
    }
  } else {
    Stage s0, s1;
    typename Stage::Offs offs = Stage::offsets(ht);
    if (nchunks > 0) {
      s0.load(rec_of(0), offs, col0b);
      if (Cf::HAS_Z) load_z(s0, 0);
      s0.store(smem, ht);
      if (Cf::HAS_Z && gz) store_z(s0, smem);
      s1.load(rec_of(last < 1 ? last : 1), offs, col0b);
      if (Cf::HAS_Z) load_z(s1, last < 1 ? last : 1);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
      s0.load(rec_of(c + 2 < last ? c + 2 : last), offs, col0b);
      if (Cf::HAS_Z) load_z(s0, c + 2 < last ? c + 2 : last);
      s1.store(smem + Cf::BUF, ht);
      if (Cf::HAS_Z && gz) store_z(s1, smem + Cf::BUF);
      __syncthreads();
      if (c + 1 >= nchunks) break;
      s1.load(rec_of(c + 3 < last ? c + 3 : last), offs, col0b);
      if (Cf::HAS_Z) load_z(s1, c + 3 < last ? c + 3 : last);
      s0.store(smem, ht);
      if (Cf::HAS_Z && gz) store_z(s0, smem);
      __syncthreads();
    }
  }

}

// ---------------------------------------------------------------------------------------------
// Wide chain kernel: bf16 records of 64-token chunks.  Each chain wave owns 32 value columns (two
// 16-column MFMA tiles), so every operand fragment it reads from LDS (-W, Q.Gamma, K'^T, P) feeds
// two MFMAs, and a workgroup of WS / 32 chain waves holds up to the full 128-column state: the
// record of a chunk is then streamed from HBM once per (sequence, head) instead of once per
// 32-column slice.  LDS tiles are unpadded and swizzled instead (WideCopy): the MFMA operand tiles
// keep the two 8-byte pieces one lane reads together, so a fragment is one 16-byte read; two
// record buffers then fit at WS = 128 (2 x 72.5 KB).
template <int DK, int DV, int WS, bool SUM, bool ZG>
struct WideCfg {
  static constexpr int C = 64;
  using R = Rec<false, DK, DV, C>;
  static_assert(R::CP == C, "64-token chunks");
  static constexpr int NT = C / 16;
  static constexpr int NWV = WS / 32;  // chain waves
  static constexpr int NH = 4;         // copy waves
  static constexpr int NTH = 64 * (NWV + NH);
  static constexpr int NC = 64 * NH;   // copy threads
  static_assert(NWV >= 1 && NWV <= 8 && WS % 32 == 0, "32 columns per chain wave");
  static constexpr int RBK = DK * 2, RBC = C * 2;  // bytes of a [..][DK] row and of a [..][C] row
  // value columns whose U~^T rows a workgroup may stream (a summary's identity columns have none)
  static constexpr int UT_ROWS = WS < DV ? WS : DV;
  static constexpr int B_NW = 0;                                  // -W        [C][DK]
  static constexpr int B_QG = B_NW + C * RBK;                     // Q.Gamma   [C][DK]   (not in summaries)
  static constexpr int B_P = B_QG + (SUM ? 0 : C * RBK);          // P         [C][C]    (not in summaries)
  static constexpr int B_KPT = B_P + (SUM ? 0 : C * RBC);         // K'^T      [DK][C]
  static constexpr int B_UT = B_KPT + DK * RBC;                   // U~^T      [UT_ROWS][C]
  static constexpr int B_GAM = B_UT + UT_ROWS * RBC;              // e^{G_last} fp32 [DK]
  // the output gate of the slice's outputs [C][ZROW bytes] where two buffers still fit (HAS_Z), else
  // the chain waves read it from global memory at the stores
  static constexpr int ZROW = WS * 2 + 16, B_Z = B_GAM + DK * 4;
  static constexpr int BUF0 = B_Z, BUFZ = B_Z + C * ZROW;
  static constexpr bool HAS_Z = ZG && 2 * BUFZ <= 163840;
  static constexpr int BUF = HAS_Z ? BUFZ : BUF0;
  static constexpr int TOTAL = 2 * BUF;
  static_assert(TOTAL <= 163840, "LDS budget of one gfx950 workgroup");
  // 16-byte copy units of one chunk's record slice
  static constexpr int U_NW = C * DK / 8, U_QG = SUM ? 0 : C * DK / 8, U_P = SUM ? 0 : C * C / 8;
  static constexpr int U_KPT = DK * C / 8, U_UT = UT_ROWS * C / 8, U_GAM = DK / 4;
  static constexpr int ZU = WS * 2 / 16;                     // output-gate units per token row
  static constexpr int ZK = (C * ZU + NC - 1) / NC;          // output-gate units per copy thread
};

// One part of a record copied by the NC copy threads in 16-byte units (NU units, UPR per row) into
// LDS rows of the same length.  Loads of units past the end repeat the last one (in bounds,
// unconditional); their stores are skipped.  NU = 0: nothing.  Layouts (MODE):
//  0  as in the record (one row, read by broadcast);
//  1  8-byte pieces XOR-swizzled: unit u of row r goes to unit u ^ ((r & 15) >> 1), its halves
//     swapped when r is odd, i.e. piece p to piece p ^ (r & 15) -- read one piece per lane;
//  2  MFMA fragment pairs: the two 8-byte pieces 8 s + g and 8 s + 4 + g (g < 4) that one lane of
//     a 16x16x32 fragment reads are stored together as 16-byte unit 4 s + g (low, high half), and
//     unit u of row r sits at u ^ (r & 7), so a fragment is one 16-byte read and the eight lanes
//     of one read cycle (rows lo = 0..7 or 8..15) hit distinct banks.  A record unit (pieces 2 a,
//     2 a + 1) lands in the low (a % 4 < 2) or high half of units 4 (a / 4) + 2 (a % 2) + {0, 1}.
template <int NC, int NU, int UPR, int GBASE, int GROW, int LBASE, int MODE>
struct WideCopy {
  static constexpr int K = NU > 0 ? (NU + NC - 1) / NC : 1;
  typedef uint32_t vec_t __attribute__((ext_vector_type(4 * K)));
  vec_t st;
  __device__ static __forceinline__ int unit(int ht, int k) {
    const int u = ht + NC * k;
    return u < NU ? u : NU - 1;
  }
  // 32-bit unit offsets formed once, as CopyPart's
  struct Off {
    uint32_t o[K];
  };
  __device__ static __forceinline__ Off offsets(int ht) {
    Off f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int u = unit(ht, k);
      f.o[k] = NU > 0 ? (uint32_t)(GBASE + (u / UPR) * GROW + 16 * (u % UPR)) : 0u;
    }
    return f;
  }
  __device__ __forceinline__ void load(const unsigned char* rec, Off& f) {
    if constexpr (NU > 0) {
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
  }
  __device__ __forceinline__ void store(unsigned char* buf, int ht) const {
    if constexpr (NU > 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (NU % NC != 0 && ht + NC * k >= NU) continue;  // only the last slot can be partial
        const int u = unit(ht, k);
        const int row = u / UPR, cu = u % UPR;
        const uint32_t a0 = st[4 * k], a1 = st[4 * k + 1], a2 = st[4 * k + 2], a3 = st[4 * k + 3];
        unsigned char* rowp = buf + LBASE + row * (UPR * 16);
        if constexpr (MODE == 0) {
          *reinterpret_cast<uint4*>(rowp + 16 * cu) = make_uint4(a0, a1, a2, a3);
        } else if constexpr (MODE == 1) {
          const int key = row & 15;
          const bool sw = (key & 1) != 0;
          *reinterpret_cast<uint4*>(rowp + 16 * (cu ^ (key >> 1))) =
              make_uint4(sw ? a2 : a0, sw ? a3 : a1, sw ? a0 : a2, sw ? a1 : a3);
        } else {
          const int key = row & 7;
          const int u0 = 4 * (cu >> 2) + 2 * (cu & 1), half = 8 * ((cu >> 1) & 1);
          *reinterpret_cast<uint2*>(rowp + 16 * (u0 ^ key) + half) = make_uint2(a0, a1);
          *reinterpret_cast<uint2*>(rowp + 16 * ((u0 + 1) ^ key) + half) = make_uint2(a2, a3);
        }
      }
    }
  }
};

// bf16 16x16x32 fragment of row r (r & 7 == lo & 7) of an LDS tile in the fragment-pair layout (MODE
// 2 above, row stride RB bytes): contraction indices 32 s + 16 (j / 4) + 4 grp + (j % 4), one
// 16-byte read of unit (4 s + grp) ^ (lo & 7).
template <int RB>
__device__ __forceinline__ bf16x8 wide_frag(const unsigned char* tile, int r, int s, int lane_key) {
  // lane_key = grp ^ (lo & 7): (4 s + grp) ^ (lo & 7) = 4 s ^ lane_key
  return *reinterpret_cast<const bf16x8*>(tile + r * RB + 16 * ((4 * s) ^ lane_key));
}

// B operand (bf16) of k-step s from accumulator tiles t0 = 2 s, t1 = 2 s + 1 of one column tile
__device__ __forceinline__ bf16x8 acc_frag(f32x4 a, f32x4 b) {
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = (__bf16)a[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) f[4 + j] = (__bf16)b[j];
  return f;
}

template <int DK, int DV, int WS, bool SUM>
__global__ __launch_bounds__(64 * (WS / 32 + 4)) void chain_wide_kernel(const ChainParams p) {
  using Cf = WideCfg<DK, DV, WS, SUM, !SUM>;
  using R = typename Cf::R;
  constexpr int C = Cf::C, NT = Cf::NT;
  constexpr int KSD = DK / 32, KSC = C / 32;
  __shared__ __align__(16) unsigned char smem[Cf::TOTAL];

  // ---- (unit, segment, slice); the slices of one (unit, segment) share an XCD (block id mod 8).
  // A summary launch has DK more columns (the identity block) and no last segment.
  constexpr int NCOL = SUM ? DV + DK : DV;
  static_assert(NCOL % WS == 0, "whole slices");
  constexpr int nsl_c = NCOL / WS;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int segs = SUM ? p.nseg - 1 : p.nseg;
  const int su = (idx / nsl_c) * 8 + xcd;
  const int slice = idx - (idx / nsl_c) * nsl_c;
  if (su >= p.units * segs) return;
  const int H = p.H;
  const int ui = su / segs, seg = su - ui * segs;
  const int n = p.order ? p.order[ui / H] : ui / H, h = ui - (ui / H) * H;
  const int unit = n * H + h;
  int64_t t_begin, t_end, first, seq0;
  if (p.nseg > 1) {  // equal-length sequences
    const int64_t s0 = (int64_t)n * p.T, s1 = s0 + p.T;
    seq0 = s0;
    t_begin = s0 + (int64_t)seg * p.seg_len * C;
    t_end = t_begin + (int64_t)p.seg_len * C < s1 ? t_begin + (int64_t)p.seg_len * C : s1;
    first = (int64_t)n * p.nch + (int64_t)seg * p.seg_len;
  } else if (p.cu) {
    int x = p.cu[n], y = p.cu[n + 1];
    x = x < 0 ? 0 : (x > p.T ? p.T : x);
    y = y < x ? x : (y > p.T ? p.T : y);
    t_begin = seq0 = x;
    t_end = y;
    first = p.chunk0[n];
  } else {
    t_begin = seq0 = (int64_t)n * p.T;
    t_end = t_begin + p.T;
    first = (int64_t)n * p.nch;
  }
  const int nchunks = (int)((t_end - t_begin + C - 1) / C);
  const int col0 = slice * WS;
  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wave < Cf::NWV;
  const int wcol = 32 * (chain ? wave : 0);  // first column of this wave within the slice
  const int ccol0 = col0 + wcol;             // first state column of this wave
  const int lkey = grp ^ (lo & 7);           // fragment-read swizzle key of this lane
  const bool idw = SUM && ccol0 >= DV;       // identity columns (U~ = 0)
  const bool no_ut = SUM && col0 >= DV;      // the whole slice is identity columns: no U~ to stream

  // ---- state in accumulator layout: Sacc[m][ct][r] = S[16 m + 4 grp + r][ccol0 + 16 ct + lo]
  f32x4 Sacc[DK / 16][2];

  auto rec_of = [&](int c) -> const unsigned char* { return p.ws + ((first + c) * H + h) * R::BYTES; };
  struct Stage {
    WideCopy<Cf::NC, Cf::U_NW, DK / 8, (int)(R::NW * 2), DK * 2, Cf::B_NW, 2> nw;
    WideCopy<Cf::NC, Cf::U_QG, DK / 8, (int)(R::QG * 2), DK * 2, Cf::B_QG, 2> qg;
    WideCopy<Cf::NC, Cf::U_P, C / 8, (int)(R::P * 2), C * 2, Cf::B_P, 2> pp;
    WideCopy<Cf::NC, Cf::U_KPT, C / 8, (int)(R::KPT * 2), C * 2, Cf::B_KPT, 2> kpt;
    WideCopy<Cf::NC, Cf::U_UT, C / 8, (int)(R::UT * 2), C * 2, Cf::B_UT, 1> ut;  // record pointer + col0 rows
    WideCopy<Cf::NC, Cf::U_GAM, Cf::U_GAM, (int)R::GAM_BYTE, 0, Cf::B_GAM, 0> gam;
    uint4 zg[Cf::ZK];
    struct Offs {
      typename decltype(nw)::Off nw;
      typename decltype(qg)::Off qg;
      typename decltype(pp)::Off pp;
      typename decltype(kpt)::Off kpt;
      typename decltype(ut)::Off ut;
      typename decltype(gam)::Off gam;
    };
  };
  // gam: one row of U_GAM units; the swizzle key of row 0 is 0, so it is stored in order
  const int ht = tid - 64 * Cf::NWV;  // copy-thread index (copy waves only)
  const int64_t col0b = (int64_t)(no_ut ? 0 : col0) * C * 2;  // first U~^T row of the slice
  // identity-column slices load a U~ slice too (col0b is then 0) and do not store it: the same loads
  // on every path keep the compiler's count of loads in flight exact
  typename Stage::Offs offs{decltype(Stage::nw)::offsets(ht), decltype(Stage::qg)::offsets(ht),
                            decltype(Stage::pp)::offsets(ht), decltype(Stage::kpt)::offsets(ht),
                            decltype(Stage::ut)::offsets(ht), decltype(Stage::gam)::offsets(ht)};
  auto stage_load = [&](Stage& st, const unsigned char* rp) {
    st.nw.load(rp, offs.nw); st.kpt.load(rp, offs.kpt); st.gam.load(rp, offs.gam);
    st.ut.load(rp + col0b, offs.ut);
    if constexpr (!SUM) { st.qg.load(rp, offs.qg); st.pp.load(rp, offs.pp); }
  };
  auto stage_store = [&](const Stage& st, unsigned char* b) {
    st.nw.store(b, ht); st.kpt.store(b, ht); st.gam.store(b, ht);
    if (!no_ut) st.ut.store(b, ht);
    if constexpr (!SUM) { st.qg.store(b, ht); st.pp.store(b, ht); }
  };
  const int ostride = H * DV;  // output elements between consecutive tokens
  // the output gate's units: ZU per row of the slice, C rows; rows past the chunk re-read its last
  // token (in bounds, never stored to o)
  auto load_z = [&](Stage& st, int c) {
    const int64_t t0 = t_begin + (int64_t)c * C;
    const int len = (int)((t_end - t0) < C ? (t_end - t0) : C);
#pragma unroll
    for (int k = 0; k < Cf::ZK; ++k) {
      int u = ht + Cf::NC * k;
      u = u < C * Cf::ZU ? u : C * Cf::ZU - 1;
      const int row = u / Cf::ZU;
      const int64_t zi = ((t0 + (row < len ? row : len - 1)) * H + h) * DV + col0 + (u % Cf::ZU) * 8;
      // unconditional, as in chain_kernel: the record buffer stands in without an output gate
      const void* zp = p.z != nullptr ? static_cast<const void*>(static_cast<const __bf16*>(p.z) + zi) : static_cast<const void*>(p.ws);
      st.zg[k] = *reinterpret_cast<const uint4*>(zp);
    }
  };
  auto store_z = [&](const Stage& st, unsigned char* b) {
#pragma unroll
    for (int k = 0; k < Cf::ZK; ++k) {
      const int u = ht + Cf::NC * k;
      if (u < C * Cf::ZU) *reinterpret_cast<uint4*>(b + Cf::B_Z + (u / Cf::ZU) * Cf::ZROW + 16 * (u % Cf::ZU)) = st.zg[k];
    }
  };
  const bool gz = !SUM && p.z != nullptr;

  // one chunk of the chain from LDS buffer `buf`.  Software-pipelined: a chain wave is the only
  // chain wave on its SIMD, so the LDS fragment reads of each group of MFMAs are issued one group
  // ahead (a sched_barrier closes every group, so the reads neither fall behind nor run further
  // ahead than the registers allow).
  auto chunk_step = [&](int c, int buf) {
    const unsigned char* b = smem + buf * Cf::BUF;
    const int64_t t0 = t_begin + (int64_t)c * C;
    const int len = (int)((t_end - t0) < C ? (t_end - t0) : C);
    const int64_t obase = (t0 * H + h) * DV;  // output element of (token t0, head h, column 0)
    if (!chain) return;
    const unsigned char* bNW = b + Cf::B_NW;
    const unsigned char* bQG = b + Cf::B_QG;
    const unsigned char* bKP = b + Cf::B_KPT;
    const unsigned char* bP = b + Cf::B_P;
    // group A (k-step sk over d_k): U += (-W) S and O^T += S^T (Q.Gamma)^T -- fragments fa, fq
    // group B (row tile m of the state): S = gamma S + K'^T U -- fragments fk
    // group C: O^T += U^T P^T -- fragments fp
    bf16x8 fa[2][NT], fq[2][NT], fk[3][KSC], fp[NT][KSC];
    auto load_a = [&](int sk, int i) {
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
        fa[i][bt] = wide_frag<Cf::RBK>(bNW, 16 * bt + lo, sk, lkey);
        if constexpr (!SUM) fq[i][bt] = wide_frag<Cf::RBK>(bQG, 16 * bt + lo, sk, lkey);
      }
    };
    auto load_b = [&](int m) {
#pragma unroll
      for (int sk = 0; sk < KSC; ++sk) fk[m % 3][sk] = wide_frag<Cf::RBC>(bKP, 16 * m + lo, sk, lkey);
    };
    auto load_c = [&]() {
#pragma unroll
      for (int bt = 0; bt < NT; ++bt)
#pragma unroll
        for (int sk = 0; sk < (16 * (bt + 1) + 31) / 32; ++sk) fp[bt][sk] = wide_frag<Cf::RBC>(bP, 16 * bt + lo, sk, lkey);
    };
    // U~ (U[bt][ct][r] = U[16 bt + 4 grp + r][16 ct + lo]; U~^T rows hold 4 consecutive tokens per
    // piece) and the first group's fragments
    f32x4 U[NT][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const unsigned char* ur = b + Cf::B_UT + (wcol + 16 * ct + lo) * Cf::RBC;
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
        if (idw) {
          U[bt][ct] = zero4();
        } else {
          const bf16x4 x = *reinterpret_cast<const bf16x4*>(ur + 8 * ((4 * bt + grp) ^ lo));
          U[bt][ct] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
        }
      }
    }
    load_a(0, 0);
    f32x4 Ot[2][NT];  // Ot[ct][bt][r] = O[token 16 bt + lo][col 16 ct + 4 grp + r]
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) Ot[ct][bt] = zero4();
    __builtin_amdgcn_sched_barrier(0);
    // group A, one k-step over d_k at a time; the old state's bf16 B fragments of that k-step are
    // formed from the accumulators as they are needed
#pragma unroll
    for (int sk = 0; sk < KSD; ++sk) {
      if (sk + 1 < KSD) {
        load_a(sk + 1, (sk + 1) & 1);
      } else {
        load_b(0);
        load_b(1);
      }
      const bf16x8 sf0 = acc_frag(Sacc[2 * sk][0], Sacc[2 * sk + 1][0]);
      const bf16x8 sf1 = acc_frag(Sacc[2 * sk][1], Sacc[2 * sk + 1][1]);
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
        U[bt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[sk & 1][bt], sf0, U[bt][0], 0, 0, 0);
        U[bt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[sk & 1][bt], sf1, U[bt][1], 0, 0, 0);
        if constexpr (!SUM) {
          Ot[0][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf0, fq[sk & 1][bt], Ot[0][bt], 0, 0, 0);
          Ot[1][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf1, fq[sk & 1][bt], Ot[1][bt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // U as B fragments (k-step over the chunk's tokens); U itself is dead after this
    bf16x8 uf[2][KSC];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int sk = 0; sk < KSC; ++sk) uf[ct][sk] = acc_frag(U[2 * sk][ct], U[2 * sk + 1][ct]);
    // group B: S = Diag(gamma) S + K'^T U, one row tile at a time, fragments two tiles ahead
    const float* gam = reinterpret_cast<const float*>(b + Cf::B_GAM);
#pragma unroll
    for (int m = 0; m < DK / 16; ++m) {
      if (m + 2 < DK / 16) load_b(m + 2);
      else if (m + 2 == DK / 16 && !SUM) load_c();
      const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * m + 4 * grp);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        Sacc[m][ct][0] *= gm.x;
        Sacc[m][ct][1] *= gm.y;
        Sacc[m][ct][2] *= gm.z;
        Sacc[m][ct][3] *= gm.w;
      }
#pragma unroll
      for (int sk = 0; sk < KSC; ++sk) {
        Sacc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[m % 3][sk], uf[0][sk], Sacc[m][0], 0, 0, 0);
        Sacc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[m % 3][sk], uf[1][sk], Sacc[m][1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SUM) return;
    // group C: O^T += U^T P^T (P lower-triangular: k-steps over tokens up to the row tile)
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
      for (int sk = 0; sk < (16 * (bt + 1) + 31) / 32; ++sk) {
        Ot[0][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uf[0][sk], fp[bt][sk], Ot[0][bt], 0, 0, 0);
        Ot[1][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uf[1][sk], fp[bt][sk], Ot[1][bt], 0, 0, 0);
      }
    }
    // output gate, stores at a wave-uniform base (the chunk's first token) plus 32-bit lane offsets
    // rebuilt here from an opaque zero, so that no per-lane 64-bit address stays live across the
    // chunk loop.  A lane holds four consecutive columns of one token in each of the two column
    // tiles; one exchange with the lane of the neighbouring column group (lane ^ 16) gives every
    // lane eight consecutive columns, so each store writes 16 bytes per lane and the four column
    // groups of a token row cover 64 contiguous bytes (two stores of 8-byte pieces covered 32).
    uint32_t zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    char* ob = reinterpret_cast<char*>(static_cast<__bf16*>(p.o) + obase);
    const char* zb = gz ? reinterpret_cast<const char*>(static_cast<const __bf16*>(p.z) + obase) : nullptr;
    const bool odd = (grp & 1) != 0;
    const int ocol = ccol0 + (odd ? 16 + 4 * (grp - 1) : 4 * grp);  // first of this lane's 8 columns
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      const int row = 16 * bt + lo;
      uint2 pk[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = ccol0 + 16 * ct + 4 * grp;
        f32x4 ov = Ot[ct][bt];
        if (gz) {
          const int zrow = row < len ? row : len - 1;
          const char* zr = Cf::HAS_Z ? reinterpret_cast<const char*>(b + Cf::B_Z + row * Cf::ZROW + (col - col0) * 2)
                                     : zb + 2u * ((uint32_t)zrow * (uint32_t)ostride + (uint32_t)col + zero);
          const uint2 zv = *reinterpret_cast<const uint2*>(zr);
          ov[0] *= __uint_as_float(zv.x << 16);
          ov[1] *= __uint_as_float(zv.x & 0xffff0000u);
          ov[2] *= __uint_as_float(zv.y << 16);
          ov[3] *= __uint_as_float(zv.y & 0xffff0000u);
        }
        pk[ct] = make_uint2(pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3]));
      }
      // even groups keep tile 0 and take the odd neighbour's tile-0 columns; odd groups the reverse
      const uint2 give = odd ? pk[0] : pk[1];
      const uint2 got = make_uint2((uint32_t)__shfl_xor((int)give.x, 16), (uint32_t)__shfl_xor((int)give.y, 16));
      const uint4 w = odd ? make_uint4(got.x, got.y, pk[1].x, pk[1].y) : make_uint4(pk[0].x, pk[0].y, got.x, got.y);
      if (row < len) *reinterpret_cast<uint4*>(ob + 2u * ((uint32_t)row * (uint32_t)ostride + (uint32_t)ocol + zero)) = w;
    }
  };
  // state snapshot after chunk c when it ends `every` tokens into the sequence (wave-uniform)
  const int rel0 = (int)(t_begin - seq0);
  auto snapshot = [&](int c) {
    const int rel_end = rel0 + (c + 1) * C;
    if (!p.states || rel_end % p.every != 0 || t_begin + (int64_t)(c + 1) * C > t_end) return;
    const int j = rel_end / p.every - 1;
    if (!p.states_by_chunk && j >= p.max_states) return;
    const int64_t slot = p.states_by_chunk ? (first + c) * H + h : (int64_t)unit * p.max_states + j;
    // a wave-uniform base and 32-bit lane offsets derived here from an opaque zero, so that the
    // compiler keeps no store addresses live across the chunk loop
    uint32_t z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const uint32_t lane_el = (4u * grp + z) * DV + ccol0 + lo;  // element offset of this lane's first value
    if (p.states_bf16) {
      char* st = reinterpret_cast<char*>(p.states) + slot * DK * DV * 2;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *reinterpret_cast<__bf16*>(st + 2u * (lane_el + (uint32_t)((16 * m + r) * DV + 16 * ct))) = (__bf16)Sacc[m][ct][r];
    } else {
      char* st = reinterpret_cast<char*>(p.states + slot * DK * DV);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *reinterpret_cast<float*>(st + 4u * (lane_el + (uint32_t)((16 * m + r) * DV + 16 * ct))) = Sacc[m][ct][r];
    }
  };

  // Chain waves compute; copy waves stream records (the loops and barriers of chain_kernel).
  const int last = nchunks - 1;
  if (chain) {
    if constexpr (SUM) {  // zero on the value columns, the identity on the extra ones
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Sacc[m][ct][r] = (idw && 16 * m + 4 * grp + r == ccol0 + 16 * ct + lo - DV) ? 1.f : 0.f;
    } else {
      const float* s0 = p.nseg > 1 ? p.sstart + ((int64_t)unit * p.nseg + seg) * DK * DV
                                   : (p.h0 ? p.h0 + (int64_t)unit * DK * DV : nullptr);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Sacc[m][ct][r] = s0 ? s0[(16 * m + 4 * grp + r) * DV + ccol0 + 16 * ct + lo] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
      chunk_step(c, 0);
      if constexpr (!SUM) snapshot(c);
      __syncthreads();
      if (c + 1 >= nchunks) break;
      chunk_step(c + 1, 1);
      if constexpr (!SUM) snapshot(c + 1);
      __syncthreads();
    }
    if constexpr (SUM) {
      float* se = p.send + ((int64_t)unit * (p.nseg - 1) + seg) * DK * (DV + DK);
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) se[(16 * m + 4 * grp + r) * (DV + DK) + ccol0 + 16 * ct + lo] = Sacc[m][ct][r];
    } else if (p.hT && seg == p.nseg - 1) {
      float* ht_ = p.hT + (int64_t)unit * DK * DV;
#pragma unroll
      for (int m = 0; m < DK / 16; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) ht_[(16 * m + 4 * grp + r) * DV + ccol0 + 16 * ct + lo] = Sacc[m][ct][r];
    }
  } else {
    Stage s0, s1;
    if (nchunks > 0) {
      stage_load(s0, rec_of(0));
      if (Cf::HAS_Z) load_z(s0, 0);
      stage_store(s0, smem);
      if (Cf::HAS_Z && gz) store_z(s0, smem);
      stage_load(s1, rec_of(last < 1 ? last : 1));
      if (Cf::HAS_Z) load_z(s1, last < 1 ? last : 1);
    }
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
      stage_load(s0, rec_of(c + 2 < last ? c + 2 : last));
      if (Cf::HAS_Z) load_z(s0, c + 2 < last ? c + 2 : last);
      stage_store(s1, smem + Cf::BUF);
      if (Cf::HAS_Z && gz) store_z(s1, smem + Cf::BUF);
      __syncthreads();
      if (c + 1 >= nchunks) break;
      stage_load(s1, rec_of(c + 3 < last ? c + 3 : last));
      if (Cf::HAS_Z) load_z(s1, c + 3 < last ? c + 3 : last);
      stage_store(s0, smem);
      if (Cf::HAS_Z && gz) store_z(s0, smem);
      __syncthreads();
    }
  }
}

template <int DK, int DV, int WS, bool SUM>
static hipError_t launch_chain_wide_impl(const ChainLaunch& L) {
  ChainParams p;
  p.ws = L.records; p.h0 = L.h0; p.o = L.o; p.hT = L.hT; p.cu = L.cu; p.chunk0 = L.chunk0; p.order = L.order;
  p.units = L.units; p.H = L.H; p.T = L.T; p.nch = L.nch; p.dv = DV;
  p.nseg = L.nseg > 1 ? L.nseg : 1; p.seg_len = L.seg_len; p.sstart = L.sstart; p.send = L.send;
  p.states = SUM ? nullptr : L.states; p.every = L.every; p.max_states = L.max_states;
  p.states_by_chunk = L.states_by_chunk ? 1 : 0;
  p.states_bf16 = L.states_bf16 ? 1 : 0;
  p.z = SUM ? nullptr : L.out_gate;
  const int64_t su = (int64_t)L.units * (SUM ? p.nseg - 1 : p.nseg);
  const int64_t grid = ((su + 7) / 8) * 8 * ((SUM ? DV + DK : DV) / WS);
  if (su <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((chain_wide_kernel<DK, DV, WS, SUM>), dim3((unsigned)grid),
                     dim3(WideCfg<DK, DV, WS, SUM, !SUM>::NTH), 0, (hipStream_t)L.stream, p);
  return hipGetLastError();
}

// Wide instances (bf16, chunk 64): value slices of 32, 64 or 128 columns (up to d_v); summaries of
// all d_v + d_k columns in one workgroup (one round of workgroups; the record streamed once).
#define KDA_WIDE_INSTANCES(X)                                                                         \
  X(64, 64, 32, false) X(64, 64, 64, false) X(64, 128, 32, false) X(64, 128, 64, false)              \
  X(64, 128, 128, false) X(128, 64, 32, false) X(128, 64, 64, false) X(128, 128, 32, false)          \
  X(128, 128, 64, false) X(128, 128, 128, false)                                                     \
  X(64, 64, 128, true) X(64, 128, 192, true) X(128, 64, 192, true) X(128, 128, 256, true)

bool chain_wide_supported(bool f32, int dk, int dv, int chunk, int ws, bool summary) {
#define KDA_HAS(D, V, W, S) \
  if (dk == D && dv == V && ws == W && summary == S) return true;
  if (f32 || chunk != 64) return false;
  KDA_WIDE_INSTANCES(KDA_HAS)
#undef KDA_HAS
  return false;
}

static hipError_t launch_chain_wide(const ChainLaunch& L) {
#define KDA_LAUNCH(D, V, W, S) \
  if (L.dk == D && L.dv == V && L.ws == W && L.summary == S) return launch_chain_wide_impl<D, V, W, S>(L);
  KDA_WIDE_INSTANCES(KDA_LAUNCH)
#undef KDA_LAUNCH
  return hipErrorInvalidValue;
}

template <bool F32, int DK, int DV, int C, int WS, bool SUM>
static hipError_t launch_chain_impl(const ChainLaunch& L) {
  ChainParams p;
  p.ws = L.records; p.h0 = L.h0; p.o = L.o; p.hT = L.hT; p.cu = L.cu; p.chunk0 = L.chunk0; p.order = L.order;
  p.units = L.units; p.H = L.H; p.T = L.T; p.nch = L.nch; p.dv = DV;
  p.nseg = L.nseg > 1 ? L.nseg : 1; p.seg_len = L.seg_len; p.sstart = L.sstart; p.send = L.send;
  p.states = SUM ? nullptr : L.states; p.every = L.every; p.max_states = L.max_states;
  p.states_by_chunk = L.states_by_chunk ? 1 : 0;
  p.states_bf16 = L.states_bf16 ? 1 : 0;
  p.z = SUM ? nullptr : L.out_gate;
  const int64_t su = (int64_t)L.units * (SUM ? p.nseg - 1 : p.nseg);
  const int64_t grid = ((su + 7) / 8) * 8 * ((SUM ? DV + DK : DV) / WS);
  if (su <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((chain_kernel<F32, DK, DV, C, WS, SUM>), dim3((unsigned)grid),
                     dim3(ChainCfg<F32, DK, DV, C, WS, !SUM>::NTH), 0, (hipStream_t)L.stream, p);
  return hipGetLastError();
}

// Slice width: bf16 picks 32 or 16 value columns per workgroup (16 -- more workgroups -- when there
// are few (sequence, head) units); fp32 uses 16.  Segment summaries use 32 or 64 (bf16: 64 when
// 32-column slices would need more than one workgroup per CU) and 16 (fp32).
#define KDA_CHAIN_BF16(X, D, V, CC) X(false, D, V, CC, 32) X(false, D, V, CC, 16)
#define KDA_CHAIN_INSTANCES(X)                                                                                   \
  KDA_CHAIN_BF16(X, 64, 64, 16) KDA_CHAIN_BF16(X, 64, 64, 32) KDA_CHAIN_BF16(X, 64, 64, 64)                        \
  KDA_CHAIN_BF16(X, 64, 128, 16) KDA_CHAIN_BF16(X, 64, 128, 32) KDA_CHAIN_BF16(X, 64, 128, 64)                     \
  KDA_CHAIN_BF16(X, 128, 64, 16) KDA_CHAIN_BF16(X, 128, 64, 32) KDA_CHAIN_BF16(X, 128, 64, 64)                     \
  KDA_CHAIN_BF16(X, 128, 128, 16) KDA_CHAIN_BF16(X, 128, 128, 32) KDA_CHAIN_BF16(X, 128, 128, 64)                  \
  KDA_CHAIN_F32(X)
#define KDA_CHAIN_F32(X)                                                                                         \
  X(true, 64, 64, 16, 16) X(true, 64, 64, 32, 16) X(true, 64, 64, 64, 16)                                         \
  X(true, 64, 128, 16, 16) X(true, 64, 128, 32, 16) X(true, 64, 128, 64, 16)                                      \
  X(true, 128, 64, 16, 16) X(true, 128, 64, 32, 16) X(true, 128, 64, 64, 16)                                      \
  X(true, 128, 128, 16, 16) X(true, 128, 128, 32, 16) X(true, 128, 128, 64, 16)
#define KDA_CHAIN_SUMMARY_INSTANCES(X)                                                                           \
  X(false, 64, 64, 16, 32) X(false, 64, 64, 32, 32) X(false, 64, 64, 64, 32)                                      \
  X(false, 64, 128, 16, 32) X(false, 64, 128, 32, 32) X(false, 64, 128, 64, 32)                                   \
  X(false, 128, 64, 16, 32) X(false, 128, 64, 32, 32) X(false, 128, 64, 64, 32)                                   \
  X(false, 128, 128, 16, 32) X(false, 128, 128, 32, 32) X(false, 128, 128, 64, 32)                                \
  X(false, 64, 64, 16, 64) X(false, 64, 64, 32, 64) X(false, 64, 64, 64, 64)                                      \
  X(false, 64, 128, 16, 64) X(false, 64, 128, 32, 64) X(false, 64, 128, 64, 64)                                   \
  X(false, 128, 64, 16, 64) X(false, 128, 64, 32, 64) X(false, 128, 64, 64, 64)                                   \
  X(false, 128, 128, 16, 64) X(false, 128, 128, 32, 64) X(false, 128, 128, 64, 64)                                \
  KDA_CHAIN_F32(X)

hipError_t launch_chain(const ChainLaunch& L) {
  if (L.wide) return launch_chain_wide(L);
  if (L.summary) {
#define KDA_LAUNCH(F, D, V, CC, W)                                                       \
  if (L.f32 == F && L.dk == D && L.dv == V && L.chunk == CC && L.ws == W && L.nseg > 1) \
    return launch_chain_impl<F, D, V, CC, W, true>(L);
    KDA_CHAIN_SUMMARY_INSTANCES(KDA_LAUNCH)
#undef KDA_LAUNCH
    return hipErrorInvalidValue;
  }
#define KDA_LAUNCH(F, D, V, CC, W) \
  if (L.f32 == F && L.dk == D && L.dv == V && L.chunk == CC && L.ws == W) return launch_chain_impl<F, D, V, CC, W, false>(L);
  KDA_CHAIN_INSTANCES(KDA_LAUNCH)
#undef KDA_LAUNCH
  return hipErrorInvalidValue;
}

// Start states of the segments of one (sequence, head), in fp32: S(0) = h0 (or 0),
// S(g + 1) = M_g S(g) + b_g, with [b_g | M_g] read from the summary launch's output.  One workgroup
// per (sequence, head, 16 value columns): d_k / 16 waves, each owning 16 rows of S(g + 1) as one
// 16x16 fp32 MFMA accumulator tile, A = M_g (staged in LDS), B = S(g) (in LDS).  While the waves
// multiply, every thread already loads its share of M_{g+1} and its b_{g+1} elements into
// registers (M_{g+1} stored into the other M buffer after the step), so a step waits on no global
// load.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void segment_combine_kernel(const float* __restrict__ h0,
                                                              const float* __restrict__ send,
                                                              float* __restrict__ sstart, int units, int nseg) {
  constexpr int CW = 16, MS = DK + 4, SE = DV + DK, NSL = DV / CW;
  constexpr int NTHC = 64 * (DK / 16);   // one wave per 16-row tile of S(g + 1)
  constexpr int MV = DK * DK / 4 / NTHC; // float4 of M_g per thread
  constexpr int RT = 1;                  // 16-row tiles per wave
  __shared__ __align__(16) float Ms[2][DK * MS];
  __shared__ __align__(16) float Ss[DK * CW];
  const int unit = blockIdx.x / NSL, col0 = (blockIdx.x % NSL) * CW;
  if (unit >= units) return;
  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, grp = lane >> 4, wave = tid >> 6;
  const float* hu = h0 ? h0 + (int64_t)unit * DK * DV : nullptr;
  float* st = sstart + (int64_t)unit * nseg * DK * DV;
  const float* se0 = send + (int64_t)unit * (nseg - 1) * DK * SE;
  // M_g, one float4 per (row, 4 columns): thread tid takes units tid + NTHC i, i.e. row
  // tid / (DK / 4) + 1024 i / DK, columns 4 (tid % (DK / 4)) ..
  const int mr = tid / (DK / 4), mj = 4 * (tid % (DK / 4));
  constexpr int MRS = NTHC / (DK / 4);  // rows between a thread's units
  // S(0) = h0 (or 0) into Ss and sstart[0]
  for (int e = tid; e < DK * CW; e += NTHC) {
    const int r = e / CW, c = e % CW;
    const float x = hu ? hu[r * DV + col0 + c] : 0.f;
    Ss[e] = x;
    st[r * DV + col0 + c] = x;
  }
  f32x4 mv[MV];
#pragma unroll
  for (int i = 0; i < MV; ++i) mv[i] = *reinterpret_cast<const f32x4*>(se0 + (mr + MRS * i) * SE + DV + mj);
#pragma unroll
  for (int i = 0; i < MV; ++i) *reinterpret_cast<f32x4*>(&Ms[0][(mr + MRS * i) * MS + mj]) = mv[i];
  // b_g rows 16 (RT wave + t) + 4 grp + r, column lo: this thread's accumulator elements
  f32x4 bv[RT];
  auto load_b = [&](const float* se) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[t][r] = se[(16 * (RT * wave + t) + 4 * grp + r) * SE + col0 + lo];
  };
  load_b(se0);
  __syncthreads();
  for (int g = 0; g + 1 < nseg; ++g) {
    // acc = b_g (loaded during the previous step), then += M_g S(g)
    f32x4 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = bv[t];
    {  // M_{g+1} and b_{g+1} (the last step reloads segment g: in bounds, never used)
      const float* sn1 = se0 + (int64_t)(g + 2 < nseg ? g + 1 : g) * DK * SE;
      load_b(sn1);
#pragma unroll
      for (int i = 0; i < MV; ++i) mv[i] = *reinterpret_cast<const f32x4*>(sn1 + (mr + MRS * i) * SE + DV + mj);
    }
    const float* m = Ms[g & 1];
#pragma unroll 8
    for (int ks = 0; ks < DK / 4; ++ks) {
      const float b = Ss[(4 * ks + grp) * CW + lo];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float a = m[(16 * (RT * wave + t) + lo) * MS + 4 * ks + grp];
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();  // every read of S(g) and M_g is done
    float* sn = st + (int64_t)(g + 1) * DK * DV;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (RT * wave + t) + 4 * grp + r;
        Ss[row * CW + lo] = acc[t][r];
        sn[row * DV + col0 + lo] = acc[t][r];
      }
    if (g + 2 < nseg) {
      float* mn = Ms[(g + 1) & 1];
#pragma unroll
      for (int i = 0; i < MV; ++i) *reinterpret_cast<f32x4*>(mn + (mr + MRS * i) * MS + mj) = mv[i];
    }
    __syncthreads();
  }
}

hipError_t launch_segment_combine(const float* h0, const float* send, float* sstart, int units, int nseg, int dk,
                                  int dv, void* stream) {
  if (units <= 0 || nseg < 2) return hipErrorInvalidValue;
#define KDA_COMB(D, V)                                                                                      \
  if (dk == D && dv == V) {                                                                                 \
    hipLaunchKernelGGL((segment_combine_kernel<D, V>), dim3(units * (V / 16)), dim3(64 * (D / 16)), 0, (hipStream_t)stream, \
                       h0, send, sstart, units, nseg);                                                      \
    return hipGetLastError();                                                                               \
  }
  KDA_COMB(64, 64) KDA_COMB(64, 128) KDA_COMB(128, 64) KDA_COMB(128, 128)
#undef KDA_COMB
  return hipErrorInvalidValue;
}

}  // namespace kda
