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
// This is pure HBM streaming (about 0.9 flop per byte).  Value columns of the state evolve
// independently (the gate acts on rows), so a (sequence, head) is split over NS workgroups by
// value-column slices: more, smaller workgroups interleave their read and write phases better.
// Each of the 256 threads holds RPT rows x 4 columns of its slice in registers (float4 accesses,
// non-temporal: the state is read and written once per step), reduces its partial column sums
// across row groups with cross-lane shuffles and one LDS exchange between the four waves, then
// writes back.
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

template <bool F32, int DK, int DV, int NS>
__global__ __launch_bounds__(256) void decode_step_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                          const void* __restrict__ v, const void* __restrict__ g,
                                                          const void* __restrict__ beta, float* __restrict__ state,
                                                          void* __restrict__ o, const DecodeFusion fu) {
  constexpr int DW = DV / NS;      // value columns of this workgroup's slice
  constexpr int C4 = DW / 4;       // threads across one slice row (float4 each)
  constexpr int RG = 256 / C4;     // row groups
  constexpr int RPT = DK / RG;     // rows per thread
  static_assert(RG * C4 == 256 && RPT * RG == DK && C4 <= 64, "shape");

  __shared__ float s_k[DK], s_q[DK], s_a[DK];
  __shared__ float s_part[4][2][DW];  // per-wave partial p and r
  __shared__ float s_kq[4], s_kk[4], s_qq[4];

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
  for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(S4 + (rg + RG * i) * RS4 + c4);
  __syncthreads();
  // normalisation factors of k and q (1 when off)
  float kn = 1.f, qn = 1.f;
  if (fu.normalize) {
    kn = __builtin_amdgcn_rsqf(s_kk[0] + s_kk[1] + s_kk[2] + s_kk[3] + 1e-12f);
    qn = __builtin_amdgcn_rsqf(s_qq[0] + s_qq[1] + s_qq[2] + s_qq[3] + 1e-12f);
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
  const float kqa = (s_kq[0] + s_kq[1] + s_kq[2] + s_kq[3]) * (kn * qn);
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = 4 * c4 + j;
    const float pp = s_part[0][0][col] + s_part[1][0][col] + s_part[2][0][col] + s_part[3][0][col];
    u[j] = b * (ldg<F32>(v, vec_v + col) - pp);
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 4 * c4 + j;
      const float rr = s_part[0][1][col] + s_part[1][1][col] + s_part[2][1][col] + s_part[3][1][col];
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
  constexpr int NS = DV == 128 ? 2 : 1;  // value-column slices per (sequence, head)
  DecodeFusion fu;
  fu.gate_scale = a.fusion.gate_scale;
  fu.normalize = a.fusion.normalize_qk ? 1 : 0;
  fu.z = a.fusion.out_gate;
  hipLaunchKernelGGL((decode_step_kernel<F32, DK, DV, NS>), dim3(a.units * NS), dim3(256), 0, (hipStream_t)a.stream,
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
