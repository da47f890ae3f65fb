// C ABI of libkda.so: argument validation, then launches on the caller's stream.
// Declarations and the contract of every entry point are in include/kda.h.
#include <stdint.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

// Fixed device scratch of kda_chunked_forward_noalloc: the per-chunk records and segment states that
// kda_chunked_forward keeps in the caller's workspace.  One copy lives on every GPU the library runs
// on, from the library's first use there until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up once per device
// (scratch_address) and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (NULL: not looked up yet)

// Device address of `scratch` on the current device, or NULL if the runtime cannot give it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#ifdef KDA_DEBUG_CHECKS
}  // namespace

// Debug build: the input envelope (-5 <= g <= 0, 0 <= beta <= 1, finite) checked on the GPU before a
// call enqueues its work.  `envelope_flag` is raised by any thread that finds a violation (plain
// stores of the same value; no atomics), cleared by a one-thread kernel before each check.
static __device__ int envelope_flag;

__global__ void envelope_clear_kernel(int* flag) {
  if (threadIdx.x == 0) flag[threadIdx.x] = 0;
}

// g [n_g] (log-decays; n_g = 0 skips them) then beta [n_b]: bf16 bits or fp32
__global__ void envelope_kernel(const void* g, const void* beta, int64_t n_g, int64_t n_b, int f32, int* flag) {
  bool bad = false;
  const int64_t n = n_g + n_b, step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
    const bool isg = i < n_g;
    const int64_t j = isg ? i : i - n_g;
    const void* base = isg ? g : beta;
    const float x = f32 ? static_cast<const float*>(base)[j]
                        : __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[j] << 16);
    const bool ok = isg ? (x >= -5.f && x <= 0.f) : (x >= 0.f && x <= 1.f);  // false for NaN
    bad = bad || !ok;
  }
  if (bad) flag[0] = 1;
}

namespace {
std::mutex g_flag_mu;
void* g_flag[kMaxDevices];  // device address of `envelope_flag` on each device

int* flag_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (!g_flag[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(envelope_flag)) != hipSuccess || !p) return nullptr;
    g_flag[dev] = p;
  }
  return static_cast<int*>(g_flag[dev]);
}
#endif

// The debug build's envelope check of g (when it holds log-decays: not a fused gate's
// pre-activation) and beta over `tokens` token-heads x H; the release build checks nothing.
// KDA_OK, KDA_ERR_ENVELOPE, or KDA_ERR_HIP.
kda_status envelope_check(const void* g, const void* beta, int64_t tokens, int H, int d_k, bool f32,
                          bool g_is_log_decay, void* hip_stream) {
#ifdef KDA_DEBUG_CHECKS
  if (tokens <= 0) return KDA_OK;
  int* flag = flag_address();
  if (!flag) return KDA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t n_g = g_is_log_decay ? tokens * H * d_k : 0, n_b = tokens * H;
  const int64_t blocks = (n_g + n_b + 255) / 256;
  hipLaunchKernelGGL(envelope_clear_kernel, dim3(1), dim3(64), 0, s, flag);
  hipLaunchKernelGGL(envelope_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s, g, beta, n_g,
                     n_b, f32 ? 1 : 0, flag);
  int raised = 0;
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyAsync(&raised, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return KDA_ERR_HIP;
  return raised ? KDA_ERR_ENVELOPE : KDA_OK;
#else
  (void)g; (void)beta; (void)tokens; (void)H; (void)d_k; (void)f32; (void)g_is_log_decay; (void)hip_stream;
  return KDA_OK;
#endif
}
bool dim_ok(int d) { return d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }

// Shared checks of the two prefill entry points (everything except the batch geometry).
kda_status check_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta, const float* h0,
                         const void* o, const float* hT, int tokens, int H, int d_k, int d_v, int chunk,
                         kda_dtype dt) {
  if (H <= 0 || d_k <= 0 || d_v <= 0 || chunk <= 0 || tokens < 0) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (tokens > 0) {
    if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) || !aligned16(o))
      return KDA_ERR_INVALID_ARG;
  }
  if ((h0 && !aligned16(h0)) || (hT && !aligned16(hT))) return KDA_ERR_INVALID_ARG;
  if (!dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
  if (!kda::chunked_forward_supported(dt == KDA_F32, d_k, d_v, chunk)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

// Fused steps: a gate scale in (0, 5] with a gate pre-activation, aligned pointers.  Fills the
// internal description and returns the pointer the kernels read as g.
bool fusion_ok(const kda_fusion* f, const void* g, kda::Fusion& out, const void*& g_eff) {
  out = kda::Fusion();
  g_eff = g;
  if (!f) return true;
  if (f->gate_x) {
    if (!(f->gate_scale > 0.f && f->gate_scale <= 5.f) || !aligned16(f->gate_x)) return false;
    out.gate_scale = f->gate_scale;
    g_eff = f->gate_x;
  }
  if (f->out_gate && !aligned16(f->out_gate)) return false;
  out.normalize_qk = f->normalize_qk != 0;
  out.out_gate = f->out_gate;
  return true;
}

// Snapshot buffer and interval: a 16-byte-aligned buffer and a positive multiple of the chunk.
bool states_ok(const float* states, int every, int chunk) {
  return aligned16(states) && every > 0 && chunk > 0 && every % chunk == 0;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case KDA_ERR_WORKSPACE: return "workspace too small";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_ENVELOPE: return "g or beta outside the documented envelope (debug build)";
  }
  return "unknown status";
}

int kda_version(void) { return 200; }

int kda_debug_checks(void) {
#ifdef KDA_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

size_t kda_chunked_forward_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt) {
  if (B <= 0 || T < 0 || H <= 0 || !chunk_ok(chunk) || (dt != KDA_F32 && dt != KDA_BF16)) return 0;
  const int64_t max_chunks = (int64_t)B * ((T + chunk - 1) / chunk);
  return kda::chunked_forward_workspace(dt == KDA_F32, d_k, d_v, chunk, max_chunks, H, B, false);
}

size_t kda_chunked_forward_varlen_workspace_bytes(int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v,
                                                  int chunk, kda_dtype dt) {
  (void)max_seqlen;
  if (num_seqs <= 0 || T_total < 0 || H <= 0 || !chunk_ok(chunk) || (dt != KDA_F32 && dt != KDA_BF16)) return 0;
  const int64_t max_chunks = (int64_t)T_total / chunk + num_seqs;
  return kda::chunked_forward_workspace(dt == KDA_F32, d_k, d_v, chunk, max_chunks, H, num_seqs, true);
}

kda_status kda_chunked_forward_plan(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt,
                                    int* value_slice, int* segments, int* segment_chunks, int* summary_slice) {
  if (B <= 0 || T < 0 || H <= 0 || chunk <= 0 || (dt != KDA_F32 && dt != KDA_BF16)) return KDA_ERR_INVALID_ARG;
  if (!dim_ok(d_k) || !dim_ok(d_v) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
  if (!kda::chunked_forward_supported(dt == KDA_F32, d_k, d_v, chunk)) return KDA_ERR_UNSUPPORTED;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda::ChainPlan pl = kda::chain_plan(dt == KDA_F32, (int64_t)B * H, (T + chunk - 1) / chunk, d_k, d_v, chunk, false);
  if (value_slice) *value_slice = pl.ws;
  if (segments) *segments = pl.nseg;
  if (segment_chunks) *segment_chunks = pl.nseg > 1 ? pl.seg_len : 0;
  if (summary_slice) *summary_slice = pl.nseg > 1 ? pl.sum_ws : 0;
  return KDA_OK;
}

namespace {
bool workspace_ok(void* ws, size_t have, size_t need) {
  if (need == 0) return true;
  return ws != nullptr && have >= need && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0;
}
}  // namespace

}  // extern "C"

namespace {
// noalloc: the fixed device scratch stands in for the caller's workspace (workspace is ignored).
kda_status chunked_forward_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                const float* h0, void* o, float* hT, float* states, int state_every,
                                const kda_fusion* fusion, int B, int T, int H, int d_k, int d_v, int chunk,
                                kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream,
                                bool noalloc = false) {
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  kda::Fusion fu;
  const void* g_eff = g;
  if (!fusion_ok(fusion, g, fu, g_eff)) return KDA_ERR_INVALID_ARG;
  const kda_status st = check_prefill(q, k, v, g_eff, beta, h0, o, hT, B * T, H, d_k, d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (states && !states_ok(states, state_every, chunk)) return KDA_ERR_INVALID_ARG;
  if (B == 0) return KDA_OK;
  if (T == 0 && !hT) return KDA_OK;
  const size_t need = kda_chunked_forward_workspace_bytes(B, T, H, d_k, d_v, chunk, dt);
  if (noalloc) {
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      if (!(workspace = scratch_address())) return KDA_ERR_HIP;
      workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (!workspace_ok(workspace, workspace_bytes, need)) return KDA_ERR_WORKSPACE;
  if (const kda_status e =
          envelope_check(g_eff, beta, (int64_t)B * T, H, d_k, dt == KDA_F32, fu.gate_scale == 0.f, hip_stream))
    return e;
  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g_eff; a.beta = beta;
  a.h0 = h0; a.o = o; a.hT = hT;
  a.cu_seqlens = nullptr;
  a.num_seqs = B;
  a.T = T;
  a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk;
  a.f32 = dt == KDA_F32;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = hip_stream;
  a.fusion = fu;
  if (states && T / state_every > 0) {
    a.states = states;
    a.state_every = state_every;
    a.max_states = T / state_every;
  }
  return kda::launch_chunked_forward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
}  // namespace

extern "C" {

kda_status kda_chunked_forward_ex(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                  const float* h0, void* o, float* hT, float* states, int state_every,
                                  const kda_fusion* fusion, int B, int T, int H, int d_k, int d_v, int chunk,
                                  kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return chunked_forward_impl(q, k, v, g, beta, h0, o, hT, states, state_every, fusion, B, T, H, d_k, d_v, chunk, dt,
                              workspace, workspace_bytes, hip_stream);
}

kda_status kda_chunked_forward_with_states(const void* q, const void* k, const void* v, const void* g,
                                           const void* beta, const float* h0, void* o, float* hT, float* states,
                                           int state_every, int B, int T, int H, int d_k, int d_v, int chunk,
                                           kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return chunked_forward_impl(q, k, v, g, beta, h0, o, hT, states, state_every, nullptr, B, T, H, d_k, d_v, chunk, dt,
                              workspace, workspace_bytes, hip_stream);
}

kda_status kda_chunked_forward_fused(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                     const float* h0, void* o, float* hT, const kda_fusion* fusion, int B, int T,
                                     int H, int d_k, int d_v, int chunk, kda_dtype dt, void* workspace,
                                     size_t workspace_bytes, void* hip_stream) {
  return chunked_forward_impl(q, k, v, g, beta, h0, o, hT, nullptr, 0, fusion, B, T, H, d_k, d_v, chunk, dt,
                              workspace, workspace_bytes, hip_stream);
}

kda_status kda_chunked_forward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v, int chunk,
                               kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return kda_chunked_forward_with_states(q, k, v, g, beta, h0, o, hT, nullptr, 0, B, T, H, d_k, d_v, chunk, dt,
                                         workspace, workspace_bytes, hip_stream);
}

kda_status kda_chunked_forward_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                       const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                       int chunk, kda_dtype dt, void* hip_stream) {
  return chunked_forward_impl(q, k, v, g, beta, h0, o, hT, nullptr, 0, nullptr, B, T, H, d_k, d_v, chunk, dt, nullptr,
                              0, hip_stream, true);
}

kda_status kda_chunked_forward_profiled(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                        const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                        int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                                        void* hip_stream, float* kernel_ms) {
  if (!kernel_ms) return KDA_ERR_INVALID_ARG;
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda_status st = check_prefill(q, k, v, g, beta, h0, o, hT, B * T, H, d_k, d_v, chunk, dt);
  if (st != KDA_OK) return st;
  kernel_ms[0] = kernel_ms[1] = 0.f;
  if (B == 0 || (T == 0 && !hT)) return KDA_OK;
  if (!workspace_ok(workspace, workspace_bytes, kda_chunked_forward_workspace_bytes(B, T, H, d_k, d_v, chunk, dt)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e = envelope_check(g, beta, (int64_t)B * T, H, d_k, dt == KDA_F32, true, hip_stream)) return e;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  for (int i = 0; i < 3; ++i)
    if (hipEventCreate(&ev[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return KDA_ERR_HIP;
    }
  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.h0 = h0; a.o = o; a.hT = hT;
  a.cu_seqlens = nullptr;
  a.num_seqs = B;
  a.T = T;
  a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk;
  a.f32 = dt == KDA_F32;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = hip_stream;
  a.events = ev;
  bool ok = kda::launch_chunked_forward(a) == hipSuccess && hipEventSynchronize(ev[2]) == hipSuccess &&
            hipEventElapsedTime(&kernel_ms[0], ev[0], ev[1]) == hipSuccess &&
            hipEventElapsedTime(&kernel_ms[1], ev[1], ev[2]) == hipSuccess;
  for (int i = 0; i < 3; ++i) (void)hipEventDestroy(ev[i]);
  return ok ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunked_forward_varlen_ex(const void* q, const void* k, const void* v, const void* g,
                                         const void* beta, const float* h0, void* o, float* hT, float* states,
                                         int state_every, const kda_fusion* fusion, const int32_t* cu_seqlens,
                                         int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v, int chunk,
                                         kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (num_seqs < 0 || T_total < 0 || max_seqlen < 0) return KDA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!cu_seqlens || max_seqlen > T_total)) return KDA_ERR_INVALID_ARG;
  if ((int64_t)num_seqs * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  kda::Fusion fu;
  const void* g_eff = g;
  if (!fusion_ok(fusion, g, fu, g_eff)) return KDA_ERR_INVALID_ARG;
  const kda_status st = check_prefill(q, k, v, g_eff, beta, h0, o, hT, T_total, H, d_k, d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (states && !states_ok(states, state_every, chunk)) return KDA_ERR_INVALID_ARG;
  if (num_seqs == 0) return KDA_OK;
  if (!workspace_ok(workspace, workspace_bytes,
                    kda_chunked_forward_varlen_workspace_bytes(num_seqs, T_total, max_seqlen, H, d_k, d_v, chunk, dt)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e =
          envelope_check(g_eff, beta, T_total, H, d_k, dt == KDA_F32, fu.gate_scale == 0.f, hip_stream))
    return e;
  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g_eff; a.beta = beta;
  a.h0 = h0; a.o = o; a.hT = hT;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.T = T_total;
  a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk;
  a.f32 = dt == KDA_F32;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = hip_stream;
  a.fusion = fu;
  if (states && max_seqlen / state_every > 0) {
    a.states = states;
    a.state_every = state_every;
    a.max_states = max_seqlen / state_every;
  }
  return kda::launch_chunked_forward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunked_forward_varlen_with_states(const void* q, const void* k, const void* v, const void* g,
                                                  const void* beta, const float* h0, void* o, float* hT,
                                                  float* states, int state_every, const int32_t* cu_seqlens,
                                                  int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v,
                                                  int chunk, kda_dtype dt, void* workspace, size_t workspace_bytes,
                                                  void* hip_stream) {
  return kda_chunked_forward_varlen_ex(q, k, v, g, beta, h0, o, hT, states, state_every, nullptr, cu_seqlens,
                                       num_seqs, T_total, max_seqlen, H, d_k, d_v, chunk, dt, workspace,
                                       workspace_bytes, hip_stream);
}

kda_status kda_chunked_forward_mxfp8(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                     const void* v, const void* v_scale, const void* g, const void* beta,
                                     const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                     int chunk, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda_status st = check_prefill(q, k, v, g, beta, h0, o, hT, B * T, H, d_k, d_v, chunk, KDA_BF16);
  if (st != KDA_OK) return st;
  if ((int64_t)B * T > 0 && (!q_scale || !k_scale || !v_scale)) return KDA_ERR_INVALID_ARG;
  if (B == 0) return KDA_OK;
  if (T == 0 && !hT) return KDA_OK;
  if (!workspace_ok(workspace, workspace_bytes, kda_chunked_forward_workspace_bytes(B, T, H, d_k, d_v, chunk, KDA_BF16)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e = envelope_check(g, beta, (int64_t)B * T, H, d_k, false, true, hip_stream)) return e;
  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.q_scale = static_cast<const uint8_t*>(q_scale);
  a.k_scale = static_cast<const uint8_t*>(k_scale);
  a.v_scale = static_cast<const uint8_t*>(v_scale);
  a.h0 = h0; a.o = o; a.hT = hT;
  a.cu_seqlens = nullptr;
  a.num_seqs = B;
  a.T = T;
  a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk;
  a.f32 = false;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = hip_stream;
  return kda::launch_chunked_forward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunked_forward_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const float* h0, void* o, float* hT, const int32_t* cu_seqlens, int num_seqs,
                                      int T_total, int max_seqlen, int H, int d_k, int d_v, int chunk, kda_dtype dt,
                                      void* workspace, size_t workspace_bytes, void* hip_stream) {
  return kda_chunked_forward_varlen_with_states(q, k, v, g, beta, h0, o, hT, nullptr, 0, cu_seqlens, num_seqs,
                                                T_total, max_seqlen, H, d_k, d_v, chunk, dt, workspace,
                                                workspace_bytes, hip_stream);
}

size_t kda_chunked_backward_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt) {
  if (B <= 0 || T < 0 || H <= 0 || (dt != KDA_F32 && dt != KDA_BF16)) return 0;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return 0;
  return kda::chunked_backward_workspace(dt == KDA_F32, d_k, d_v, chunk, B, T, H, false);
}

namespace {
// Checks shared by the two backward entry points (everything except the batch geometry).
kda_status check_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const float* h0, const void* d_o, const float* dhT, void* dq, void* dk, void* dv, void* dg,
                          void* dbeta, float* dh0, int tokens, int H, int d_k, int d_v, int chunk, kda_dtype dt) {
  // the forward's checks (inputs, h0; d_o in place of o), then the gradient buffers
  const kda_status st = check_prefill(q, k, v, g, beta, h0, d_o, dhT, tokens, H, d_k, d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (tokens > 0) {
    if (!dq || !dk || !dv || !dg || !dbeta) return KDA_ERR_INVALID_ARG;
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg) || !aligned16(dbeta))
      return KDA_ERR_INVALID_ARG;
  }
  if (dh0 && !aligned16(dh0)) return KDA_ERR_INVALID_ARG;
  if (!kda::chunked_backward_supported(dt == KDA_F32, d_k, d_v, chunk)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}
}  // namespace

kda_status kda_chunked_backward(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                const float* h0, const void* d_o, const float* dhT, void* dq, void* dk, void* dv,
                                void* dg, void* dbeta, float* dh0, int B, int T, int H, int d_k, int d_v, int chunk,
                                kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda_status st = check_backward(q, k, v, g, beta, h0, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, B * T, H, d_k,
                                       d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (B == 0 || (T == 0 && !dh0)) return KDA_OK;
  if (!workspace_ok(workspace, workspace_bytes, kda_chunked_backward_workspace_bytes(B, T, H, d_k, d_v, chunk, dt)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e = envelope_check(g, beta, (int64_t)B * T, H, d_k, dt == KDA_F32, true, hip_stream)) return e;
  kda::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dO = d_o; a.dhT = dhT;
  a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
  a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.f32 = dt == KDA_F32;
  a.workspace = workspace;
  a.stream = hip_stream;
  return kda::launch_chunked_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunked_forward_train_saved_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt) {
  if (B <= 0 || T < 0 || H <= 0 || (dt != KDA_F32 && dt != KDA_BF16)) return 0;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return 0;
  return kda::chunked_backward_saved_bytes(dt == KDA_F32, d_k, d_v, chunk, B, T, H, false);
}

size_t kda_chunked_backward_saved_workspace_bytes(int B, int T, int H, int d_k, int d_v, int chunk, kda_dtype dt) {
  if (B <= 0 || T < 0 || H <= 0 || (dt != KDA_F32 && dt != KDA_BF16)) return 0;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return 0;
  return kda::chunked_backward_own_bytes(dt == KDA_F32, d_k, d_v, chunk, B, T, H, false);
}

kda_status kda_chunked_forward_train(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                     const float* h0, void* o, float* hT, int B, int T, int H, int d_k, int d_v,
                                     int chunk, kda_dtype dt, void* saved, size_t saved_bytes, void* hip_stream) {
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda_status st = check_prefill(q, k, v, g, beta, h0, o, hT, B * T, H, d_k, d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (!kda::chunked_backward_supported(dt == KDA_F32, d_k, d_v, chunk)) return KDA_ERR_UNSUPPORTED;
  if (B == 0 || (T == 0 && !hT)) return KDA_OK;
  if (!workspace_ok(saved, saved_bytes, kda_chunked_forward_train_saved_bytes(B, T, H, d_k, d_v, chunk, dt)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e = envelope_check(g, beta, (int64_t)B * T, H, d_k, dt == KDA_F32, true, hip_stream)) return e;
  kda::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0;
  a.dO = nullptr; a.dhT = nullptr;
  a.dq = a.dk_out = a.dv_out = a.dg = a.dbeta = nullptr; a.dh0 = nullptr;
  a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.f32 = dt == KDA_F32;
  a.workspace = nullptr;
  a.stream = hip_stream;
  return kda::launch_forward_train(a, saved, o, hT) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunked_backward_saved(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const float* h0, const void* d_o, const float* dhT, void* dq, void* dk,
                                      void* dv, void* dg, void* dbeta, float* dh0, int B, int T, int H, int d_k,
                                      int d_v, int chunk, kda_dtype dt, const void* saved, size_t saved_bytes,
                                      void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX || (int64_t)B * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda_status st = check_backward(q, k, v, g, beta, h0, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, B * T, H, d_k,
                                       d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (B == 0 || (T == 0 && !dh0)) return KDA_OK;
  if (!workspace_ok(const_cast<void*>(saved), saved_bytes,
                    kda_chunked_forward_train_saved_bytes(B, T, H, d_k, d_v, chunk, dt)) ||
      !workspace_ok(workspace, workspace_bytes, kda_chunked_backward_saved_workspace_bytes(B, T, H, d_k, d_v, chunk, dt)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e = envelope_check(g, beta, (int64_t)B * T, H, d_k, dt == KDA_F32, true, hip_stream)) return e;
  kda::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dO = d_o; a.dhT = dhT;
  a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
  a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.f32 = dt == KDA_F32;
  a.workspace = workspace;
  a.saved = saved;
  a.stream = hip_stream;
  return kda::launch_chunked_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunked_backward_varlen_workspace_bytes(int num_seqs, int T_total, int max_seqlen, int H, int d_k,
                                                   int d_v, int chunk, kda_dtype dt) {
  (void)max_seqlen;
  if (num_seqs <= 0 || T_total < 0 || H <= 0 || !chunk_ok(chunk) || (dt != KDA_F32 && dt != KDA_BF16)) return 0;
  if ((int64_t)num_seqs * H > INT32_MAX / 8) return 0;
  return kda::chunked_backward_workspace(dt == KDA_F32, d_k, d_v, chunk, num_seqs, T_total, H, true);
}

kda_status kda_chunked_backward_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                       const float* h0, const void* d_o, const float* dhT, void* dq, void* dk,
                                       void* dv, void* dg, void* dbeta, float* dh0, const int32_t* cu_seqlens,
                                       int num_seqs, int T_total, int max_seqlen, int H, int d_k, int d_v, int chunk,
                                       kda_dtype dt, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (num_seqs < 0 || T_total < 0 || max_seqlen < 0) return KDA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!cu_seqlens || max_seqlen > T_total)) return KDA_ERR_INVALID_ARG;
  if ((int64_t)num_seqs * H > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
  const kda_status st = check_backward(q, k, v, g, beta, h0, d_o, dhT, dq, dk, dv, dg, dbeta, dh0, T_total, H, d_k,
                                       d_v, chunk, dt);
  if (st != KDA_OK) return st;
  if (num_seqs == 0 || (T_total == 0 && !dh0)) return KDA_OK;
  if (!workspace_ok(workspace, workspace_bytes,
                    kda_chunked_backward_varlen_workspace_bytes(num_seqs, T_total, max_seqlen, H, d_k, d_v, chunk, dt)))
    return KDA_ERR_WORKSPACE;
  if (const kda_status e = envelope_check(g, beta, T_total, H, d_k, dt == KDA_F32, true, hip_stream)) return e;
  kda::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dO = d_o; a.dhT = dhT;
  a.dq = dq; a.dk_out = dk; a.dv_out = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
  a.cu_seqlens = cu_seqlens;
  a.B = num_seqs; a.T = T_total; a.H = H; a.dk = d_k; a.dv = d_v; a.chunk = chunk; a.f32 = dt == KDA_F32;
  a.workspace = workspace;
  a.stream = hip_stream;
  return kda::launch_chunked_backward(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step_fused(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 float* state, void* o, const kda_fusion* fusion, int B, int H, int d_k, int d_v,
                                 kda_dtype dt, void* hip_stream) {
  if (B < 0 || H <= 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_INVALID_ARG;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if ((int64_t)B * H > INT32_MAX / 2) return KDA_ERR_UNSUPPORTED;
  kda::Fusion fu;
  const void* g_eff = g;
  if (!fusion_ok(fusion, g, fu, g_eff)) return KDA_ERR_INVALID_ARG;
  if (B > 0) {
    if (!q || !k || !v || !g_eff || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g_eff) || !aligned16(beta) ||
        !aligned16(state) || !aligned16(o))
      return KDA_ERR_INVALID_ARG;
  }
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (const kda_status e = envelope_check(g_eff, beta, B, H, d_k, dt == KDA_F32, fu.gate_scale == 0.f, hip_stream))
    return e;
  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g_eff; a.beta = beta;
  a.state = state;
  a.o = o;
  a.units = B * H;
  a.dk = d_k;
  a.dv = d_v;
  a.f32 = dt == KDA_F32;
  a.stream = hip_stream;
  a.fusion = fu;
  return kda::launch_decode_step(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta, float* state,
                           void* o, int B, int H, int d_k, int d_v, kda_dtype dt, void* hip_stream) {
  return kda_decode_step_fused(q, k, v, g, beta, state, o, nullptr, B, H, d_k, d_v, dt, hip_stream);
}

}  // extern "C"
