// KDA chunked prefill on gfx950: orchestration of the three kernels, all on the caller's stream.
//
//   1. chunk_map_kernel    (packed sequences only) first chunk of every sequence, from the device
//                          offsets -- no host synchronisation
//   2. intra_chunk_kernel  gate cumulative sum + UT/WY transform of every (chunk, head), in parallel,
//                          into per-chunk records in the workspace
//   3. chain_kernel        the sequential state chain per (sequence, head, value slice); for long
//                          sequences on few heads, per segment: a summary launch, the segment
//                          start states (segment_combine_kernel), then the chain of every segment
//
// Workspace: [records: max_chunks * H * record bytes][chunk0: (num_seqs + 1) int32, and the
// sequences longest first: num_seqs int32, packed only][segment start states: units * nseg * d_k * d_v fp32][segment summaries: units * (nseg - 1) *
// d_k * (d_v + d_k) fp32], the last two only when the plan splits sequences into nseg > 1
// segments.  max_chunks bounds the number of chunks: B * ceil(T / C) for equal-length sequences,
// floor(T_total / C) + num_seqs for packed ones (each sequence adds at most one partial chunk).
#include <atomic>

#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

bool chunked_forward_supported(bool f32, int dk, int dv, int chunk) { return record_bytes(f32, dk, dv, chunk) > 0; }

static int64_t max_chunks_of(int T, int chunk, int num_seqs, bool varlen) {
  return varlen ? (int64_t)T / chunk + num_seqs : (int64_t)num_seqs * ((T + chunk - 1) / chunk);
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segments: at least kMinSegChunks chunks each, at most kMaxSeg per (sequence, head).
static constexpr int kMinSegChunks = 32, kMaxSeg = 64;

ChainPlan chain_plan(bool f32, int64_t units, int nch, int dk, int dv, int chunk, bool varlen) {
  const int cus = compute_units();
  ChainPlan pl{16, 1, 0, 0, false};
  if (!f32 && chunk == 64 && !varlen && units * (dv / 32) < cus && nch >= 2 * kMinSegChunks) {
    // segments on the wide kernel (chain waves of 32 columns, a workgroup of ws / 32 of them).
    // Unsegmented plans stay on chain_kernel: two 16-column chain waves per workgroup finish a
    // chunk sooner than one 32-column wave, and there the chunk time is the whole chain's pace.
    // Long sequences on few heads: the widest slice (each record then streamed from HBM by fewer
    // workgroups) whose segments, enough of them to fill the CUs, still hold kMinSegChunks chunks.
    for (int ws = dv; ws >= 32; ws /= 2) {
      const int64_t per = units * (dv / ws);
      int64_t nseg = (cus + per - 1) / per;
      if (nseg > kMaxSeg) nseg = kMaxSeg;
      if (ws > 32 && nseg * kMinSegChunks > nch) continue;
      if (nseg > nch / kMinSegChunks) nseg = nch / kMinSegChunks;
      if (nseg < 2) break;
      pl.ws = ws;
      pl.seg_len = (int)((nch + nseg - 1) / nseg);
      pl.nseg = (nch + pl.seg_len - 1) / pl.seg_len;
      pl.sum_ws = dk + dv;  // a summary workgroup holds the value and identity columns together
      pl.wide = true;
      return pl;
    }
  }
  if (!f32 && units * (dv / 32) >= cus) pl.ws = 32;
  // Long sequences on few heads: (sequence, head, slice) alone leave CUs idle, so split every
  // sequence into segments.  That triples the chain's work (summaries over twice the columns, then
  // the chain itself) but runs it on nseg times more workgroups.
  const int wss = f32 ? 16 : 32;
  const int64_t per = units * (dv / wss);
  if (!varlen && per < cus && nch >= 2 * kMinSegChunks) {
    int64_t nseg = (cus + per - 1) / per;
    if (nseg > nch / kMinSegChunks) nseg = nch / kMinSegChunks;
    if (nseg > kMaxSeg) nseg = kMaxSeg;
    if (nseg >= 2) {
      pl.ws = wss;
      pl.seg_len = (int)((nch + nseg - 1) / nseg);
      pl.nseg = (nch + pl.seg_len - 1) / pl.seg_len;
      // the summary has d_k more columns than the chain; where its slices of wss columns would need
      // more than one round of workgroups (one per CU: the record buffers fill the LDS), bf16
      // summaries take 64-column slices, one round at twice the work per workgroup
      pl.sum_ws = wss;
      if (!f32 && units * (int64_t)(pl.nseg - 1) * ((dv + dk) / 32) > cus) pl.sum_ws = 64;
    }
  }
  return pl;
}

size_t chunked_forward_workspace(bool f32, int dk, int dv, int chunk, int64_t max_chunks, int H, int num_seqs,
                                 bool varlen) {
  const int64_t rb = record_bytes(f32, dk, dv, chunk);
  if (rb == 0) return 0;
  size_t bytes = (size_t)(max_chunks * H * rb);
  if (varlen) bytes += al256((size_t)(num_seqs + 1) * 4) + al256((size_t)num_seqs * 4);  // chunk map, order
  const int nch = (!varlen && num_seqs > 0) ? (int)(max_chunks / num_seqs) : 0;
  const ChainPlan pl = chain_plan(f32, (int64_t)num_seqs * H, nch, dk, dv, chunk, varlen);
  if (pl.nseg > 1) {
    const size_t units = (size_t)num_seqs * H;
    bytes += al256(units * pl.nseg * dk * dv * 4) + al256(units * (pl.nseg - 1) * dk * (dv + dk) * 4);
  }
  return bytes;
}

// CUs of the current device (256 when no device can be queried), cached per device; calls from
// several host threads may query concurrently and store the same value.
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Where a packed call's chunk map sits in its workspace (after the records): the first chunk of every
// sequence [num_seqs + 1] and the sequences longest first [num_seqs].
void chunk_map_of(void* workspace, bool f32, int dk, int dv, int chunk, int64_t max_chunks, int H, int num_seqs,
                  int32_t** chunk0, int32_t** order) {
  unsigned char* c0 = static_cast<unsigned char*>(workspace) + max_chunks * H * record_bytes(f32, dk, dv, chunk);
  *chunk0 = reinterpret_cast<int32_t*>(c0);
  *order = reinterpret_cast<int32_t*>(c0 + al256((size_t)(num_seqs + 1) * 4));
}

hipError_t launch_chunked_forward(const PrefillArgs& a) {
  const bool varlen = a.cu_seqlens != nullptr;
  const int C = a.chunk;
  const int64_t rb = record_bytes(a.f32, a.dk, a.dv, C);
  if (rb == 0) return hipErrorInvalidValue;
  const int64_t max_chunks = max_chunks_of(a.T, C, a.num_seqs, varlen);
  const int nch = varlen ? 0 : (a.T + C - 1) / C;
  unsigned char* records = static_cast<unsigned char*>(a.workspace);
  int32_t* chunk0 = nullptr;
  int32_t* order = nullptr;
  hipError_t e = hipSuccess;
  if (a.events && (e = hipEventRecord(a.events[0], (hipStream_t)a.stream)) != hipSuccess) return e;
  if (varlen) {
    chunk_map_of(a.workspace, a.f32, a.dk, a.dv, C, max_chunks, a.H, a.num_seqs, &chunk0, &order);
    e = launch_chunk_map(a.cu_seqlens, a.num_seqs, a.T, C, chunk0, order, a.stream);
    if (e != hipSuccess) return e;
  }
  const int64_t items = max_chunks * a.H;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  if (items > 0) {
    IntraLaunch L;
    L.q = a.q; L.k = a.k; L.v = a.v; L.g = a.g; L.beta = a.beta;
    L.qs = a.q_scale; L.ks = a.k_scale; L.vs = a.v_scale;
    L.cu = a.cu_seqlens; L.chunk0 = chunk0; L.records = records;
    L.num_seqs = a.num_seqs; L.H = a.H; L.T = a.T; L.nch = nch;
    L.dk = a.dk; L.dv = a.dv; L.chunk = C; L.f32 = a.f32;
    L.grid = (int)items;  // one 8-wave workgroup per (chunk, head) record (bound; extra ones exit)
    L.gate_scale = a.fusion.gate_scale;
    L.normalize_qk = a.fusion.normalize_qk;
    L.stream = a.stream;
    e = launch_intra(L);
    if (e != hipSuccess) return e;
  }
  if (a.events && (e = hipEventRecord(a.events[1], (hipStream_t)a.stream)) != hipSuccess) return e;
  ChainLaunch K;
  K.records = records; K.h0 = a.h0; K.o = a.o; K.hT = a.hT; K.cu = a.cu_seqlens; K.chunk0 = chunk0; K.order = order;
  K.units = a.num_seqs * a.H; K.H = a.H; K.T = a.T; K.nch = nch;
  K.dk = a.dk; K.dv = a.dv; K.chunk = C; K.f32 = a.f32;
  const ChainPlan pl = chain_plan(a.f32, K.units, nch, a.dk, a.dv, C, varlen);
  K.wide = pl.wide;
  K.ws = pl.ws;
  K.stream = a.stream;
  K.states = a.states; K.every = a.state_every; K.max_states = a.max_states; K.states_by_chunk = a.states_by_chunk;
  K.states_bf16 = a.states_bf16;
  K.out_gate = a.fusion.out_gate;
  if (pl.nseg > 1) {
    unsigned char* seg = records + max_chunks * a.H * rb;
    float* sstart = reinterpret_cast<float*>(seg);
    float* send = reinterpret_cast<float*>(seg + al256((size_t)K.units * pl.nseg * a.dk * a.dv * 4));
    K.nseg = pl.nseg; K.seg_len = pl.seg_len; K.sstart = sstart; K.send = send;
    K.summary = true;
    K.ws = pl.sum_ws;
    if ((e = launch_chain(K)) != hipSuccess) return e;
    K.ws = pl.ws;
    if ((e = launch_segment_combine(a.h0, send, sstart, K.units, pl.nseg, a.dk, a.dv, a.stream)) != hipSuccess) return e;
    K.summary = false;
  }
  if ((e = launch_chain(K)) != hipSuccess) return e;
  if (a.events) e = hipEventRecord(a.events[2], (hipStream_t)a.stream);
  return e;
}

}  // namespace kda
