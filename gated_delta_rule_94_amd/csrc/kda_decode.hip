// KDA single-token decode step on gfx950.
//
// The fixed-size recurrent state is what makes per-token decode cost
// independent of context length (architecture blog, "Why the attention stack
// is the story"; how-K3-works page, "KDA: a fixed memory instead of a growing
// bill").  One step for one (sequence, head), with S the d_k x d_v fp32 state:
//   S' = Diag(exp(g)) S                      (channel-wise forget gate)
//   p  = S'^T k,  r = S'^T q                 (two column reductions over d_k)
//   u  = beta (v - p)                        (delta-rule correction)
//   S  = S' + k u^T,   o = S^T q = r + (k . q) u
// so the state is read once and written once, and o needs no second pass.
//
// This is pure HBM streaming (about 0.9 flop per byte).  One workgroup of 512 threads owns one
// (sequence, head): each thread holds RPT rows x 4 columns of the state in registers (float4
// accesses; a wave covers whole 512-byte state rows), reduces its partial column sums across row
// groups with cross-lane shuffles and one LDS exchange between the eight waves, then writes back.
// The state is read with ordinary loads and written with non-temporal stores (it is written once
// per step and not read again within it).  Value columns evolve independently (the gate acts on
// rows), so the kernel also takes NS > 1 column slices per (sequence, head); on the 256 x 32 x
// 128 x 128 state one whole-head workgroup with this load/store mix streamed fastest (measured on
// MI355X: 161 us per step against 192 us for two 64-column workgroups with non-temporal loads).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Optional fused steps (all off by default): gate_scale > 0 -- g holds the gate pre-activation x and
// g = -gate_scale sigmoid(x); normalize -- q and k are L2-normalised over d_k; z -- o is multiplied
// by it elementwise.
struct DecodeFusion {
  float gate_scale;
  int normalize;
  const void* z;
};

template <bool F32, int DK, int DV, int NS, int THR>
__global__ __launch_bounds__(THR) void decode_step_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                          const void* __restrict__ v, const void* __restrict__ g,
                                                          const void* __restrict__ beta, float* __restrict__ state,
                                                          void* __restrict__ o, const DecodeFusion fu) {
  constexpr int NW = THR / 64;     // waves
  constexpr int DW = DV / NS;      // value columns of this workgroup's slice
  constexpr int C4 = DW / 4;       // threads across one slice row (float4 each)
  constexpr int RG = THR / C4;     // row groups
  constexpr int RPT = DK / RG;     // rows per thread
  static_assert(RG * C4 == THR && RPT * RG == DK && C4 <= 64 && THR >= DK, "shape");

  __shared__ float s_k[DK], s_q[DK], s_a[DK];
  __shared__ float s_part[NW][2][DW];  // per-wave partial p and r
  __shared__ float s_kq[NW], s_kk[NW], s_qq[NW];

  const int unit = blockIdx.x / NS;  // b * H + h
  const int col0 = (blockIdx.x - unit * NS) * DW;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t vec_k = (int64_t)unit * DK, vec_v = (int64_t)unit * DV + col0;

  // gate, key and query of this (sequence, head); k.q (and |k|^2, |q|^2) by block reductions
  float kq = 0.f, k2 = 0.f, q2 = 0.f;
  if (tid < DK) {
    float kk = ldg<F32>(k, vec_k + tid), qq = ldg<F32>(q, vec_k + tid);
    s_k[tid] = kk;
    s_q[tid] = qq;
    const float x = ldg<F32>(g, vec_k + tid);
    s_a[tid] = __expf(fu.gate_scale > 0.f ? -fu.gate_scale * __builtin_amdgcn_rcpf(1.f + __expf(-x)) : x);
    kq = kk * qq;
    k2 = kk * kk;
    q2 = qq * qq;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off);
  if (lane == 0) s_kq[wave] = kq;
  if (fu.normalize) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      k2 += __shfl_xor(k2, off);
      q2 += __shfl_xor(q2, off);
    }
    if (lane == 0) {
      s_kk[wave] = k2;
      s_qq[wave] = q2;
    }
  }

  const int c4 = tid % C4, rg = tid / C4;
  f32x4* S4 = reinterpret_cast<f32x4*>(state + (int64_t)unit * DK * DV + col0);
  constexpr int RS4 = DV / 4;  // float4 per full state row
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = S4[(rg + RG * i) * RS4 + c4];
  __syncthreads();
  // normalisation factors of k and q (1 when off)
  float kn = 1.f, qn = 1.f;
  if (fu.normalize) {
    float kk = 1e-12f, qq = 1e-12f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      kk += s_kk[w];
      qq += s_qq[w];
    }
    kn = __builtin_amdgcn_rsqf(kk);
    qn = __builtin_amdgcn_rsqf(qq);
  }

  float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const float a = s_a[row], kr = s_k[row] * kn, qr = s_q[row] * qn;
    s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
    p[0] += s[i].x * kr; p[1] += s[i].y * kr; p[2] += s[i].z * kr; p[3] += s[i].w * kr;
    r[0] += s[i].x * qr; r[1] += s[i].y * qr; r[2] += s[i].z * qr; r[3] += s[i].w * qr;
  }
  // reduce over the row groups inside the wave (lanes differing by multiples of C4)
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] += __shfl_xor(p[j], off);
      r[j] += __shfl_xor(r[j], off);
    }
  }
  if (lane < C4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s_part[wave][0][4 * c4 + j] = p[j];
      s_part[wave][1][4 * c4 + j] = r[j];
    }
  }
  __syncthreads();
  const float b = ldg<F32>(beta, unit);
  float kqs = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) kqs += s_kq[w];
  const float kqa = kqs * (kn * qn);
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = 4 * c4 + j;
    float pp = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) pp += s_part[w][0][col];
    u[j] = b * (ldg<F32>(v, vec_v + col) - pp);
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 4 * c4 + j;
      float rr = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) rr += s_part[w][1][col];
      const float zz = fu.z ? ldg<F32>(fu.z, vec_v + col) : 1.f;
      stg<F32>(o, vec_v + col, (rr + kqa * u[j]) * zz);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float kr = s_k[rg + RG * i] * kn;
    s[i].x += kr * u[0]; s[i].y += kr * u[1]; s[i].z += kr * u[2]; s[i].w += kr * u[3];
    __builtin_nontemporal_store(s[i], S4 + (rg + RG * i) * RS4 + c4);
  }
}

template <bool F32, int DK, int DV>
static hipError_t launch_decode(const DecodeArgs& a) {
  constexpr int NS = 1, THR = 512;  // one workgroup of 512 threads per (sequence, head)
  DecodeFusion fu;
  fu.gate_scale = a.fusion.gate_scale;
  fu.normalize = a.fusion.normalize_qk ? 1 : 0;
  fu.z = a.fusion.out_gate;
  hipLaunchKernelGGL((decode_step_kernel<F32, DK, DV, NS, THR>), dim3(a.units * NS), dim3(THR), 0, (hipStream_t)a.stream,
                     a.q, a.k, a.v, a.g, a.beta, a.state, a.o, fu);
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeArgs& a) {
  const int key = (a.f32 ? 1000 : 0) + a.dk * 10 + a.dv / 64;
  switch (key) {
    case 641: return launch_decode<false, 64, 64>(a);
    case 642: return launch_decode<false, 64, 128>(a);
    case 1281: return launch_decode<false, 128, 64>(a);
    case 1282: return launch_decode<false, 128, 128>(a);
    case 1641: return launch_decode<true, 64, 64>(a);
    case 1642: return launch_decode<true, 64, 128>(a);
    case 2281: return launch_decode<true, 128, 64>(a);
    case 2282: return launch_decode<true, 128, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
