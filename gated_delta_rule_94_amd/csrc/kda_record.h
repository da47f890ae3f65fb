// Per-(chunk, head) record written by the intra-chunk kernel and read by the chain kernel.
//
// For a chunk of C tokens with chunk-local cumulative log-decay G (Gamma = e^G) the record holds
// everything the sequential state chain needs, so that nothing but the state itself is carried
// from chunk to chunk (element type E: bf16 for bf16 inputs, fp32 for fp32 inputs):
//   NW   -W = -T (K . Gamma)                    [C][DK]     (negated: the chain adds it)
//   QG   Q . Gamma                              [C][DK]
//   KPT  (K . e^{G_last - G})^T                  [DK][CP]    token-contiguous
//   P    lowerIncl(q_r . k_i e^{G_r - G_i})      [C][CP]     tiles the chain reads above the
//                                                            diagonal are written as zeros
//   UT   (T V)^T = U~^T                          [DV][C]     token-contiguous
//   GAM  e^{G_last}  (fp32)                      [DK]
// CP is the token extent of token-contraction operands (C, or 32 when a bf16 chunk of 16 must
// fill one 32-deep MFMA step; the extra columns are zero).  Records are 256-byte aligned.
#pragma once

#include <stdint.h>

namespace kda {

template <bool F32, int DK, int DV, int C>
struct Rec {
  static constexpr int CP = (!F32 && C < 32) ? 32 : C;
  static constexpr int ES = F32 ? 4 : 2;
  static constexpr int64_t NW = 0;
  static constexpr int64_t QG = NW + (int64_t)C * DK;
  static constexpr int64_t KPT = QG + (int64_t)C * DK;
  static constexpr int64_t P = KPT + (int64_t)DK * CP;
  static constexpr int64_t UT = P + (int64_t)C * CP;
  static constexpr int64_t END = UT + (int64_t)C * DV;  // elements of type E
  static constexpr int64_t GAM_BYTE = ((END * ES) + 15) & ~(int64_t)15;
  static constexpr int64_t BYTES = (GAM_BYTE + 4 * DK + 255) & ~(int64_t)255;
};

// Record size for a runtime shape (0 if unsupported).
inline int64_t record_bytes(bool f32, int dk, int dv, int chunk) {
#define KDA_REC(F, D, V, CC) \
  if (f32 == F && dk == D && dv == V && chunk == CC) return Rec<F, D, V, CC>::BYTES;
  KDA_REC(false, 64, 64, 16) KDA_REC(false, 64, 64, 32) KDA_REC(false, 64, 64, 64)
  KDA_REC(false, 64, 128, 16) KDA_REC(false, 64, 128, 32) KDA_REC(false, 64, 128, 64)
  KDA_REC(false, 128, 64, 16) KDA_REC(false, 128, 64, 32) KDA_REC(false, 128, 64, 64)
  KDA_REC(false, 128, 128, 16) KDA_REC(false, 128, 128, 32) KDA_REC(false, 128, 128, 64)
  KDA_REC(true, 64, 64, 16) KDA_REC(true, 64, 64, 32) KDA_REC(true, 64, 64, 64)
  KDA_REC(true, 64, 128, 16) KDA_REC(true, 64, 128, 32) KDA_REC(true, 64, 128, 64)
  KDA_REC(true, 128, 64, 16) KDA_REC(true, 128, 64, 32) KDA_REC(true, 128, 64, 64)
  KDA_REC(true, 128, 128, 16) KDA_REC(true, 128, 128, 32) KDA_REC(true, 128, 128, 64)
#undef KDA_REC
  return 0;
}

}  // namespace kda
