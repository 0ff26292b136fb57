// Route construction on the GPU: zigzag <-> contiguous runs by interval
// intersection, with no host round trip.
//
// Method (Relax PR #273 "fla mcore chunkwise cp stage 3", §2.1): both layouts
// are unions of global token intervals -- one interval per rank for the
// contiguous layout, two per document per rank for the zigzag layout -- so the
// whole exchange is an intersection of intervals instead of per-token index
// tensors.  The pages do this with Python integers on the host after one
// device-to-host copy of the boundaries; here one workgroup does it on the
// device, so the host never waits.
//
// Layout facts used below ("Packed Sequence 与上下文并行" §2.4, §2.5, §3.5):
//  * a padded document k of length L_k starting at token a_k is cut into 2*cp
//    chunks of c_k = L_k / (2*cp) tokens; chunk q belongs to rank q (q < cp)
//    or 2*cp-1-q (q >= cp);
//  * in rank r's zigzag share the documents come in order, each contributing
//    its chunk r then its chunk 2*cp-1-r; every earlier document contributes
//    L_j / cp rows, so document k starts at local row a_k / cp;
//  * the contiguous share of rank d is tokens [d*T/cp, (d+1)*T/cp), so in the
//    emulated contiguous buffer the row of token g is g itself.
// A zigzag segment is therefore one token interval [g0, g0 + c_k) sitting at
// emulated zigzag rows [s0, s0 + c_k) with s0 = r*T/cp + a_k/cp + h*c_k (h = 1
// for the back chunk).  Cutting it at multiples of T/cp (the contiguous ranks'
// borders) gives the route's pieces; pieces that touch in both coordinates
// inside one (source rank, destination rank) pair are merged into one run.
#include "thd_internal.h"

namespace thdcp {
namespace {

constexpr int kBuildThreads = 1024;
constexpr int kBuildWaves = kBuildThreads / 64;

// Make global-memory writes of the whole workgroup visible to all its threads.
__device__ __forceinline__ void wg_sync_global() {
  __threadfence();
  __syncthreads();
  __threadfence();
}

// Exclusive prefix sum over the workgroup.  Every thread must call it; it
// returns the thread's exclusive offset and the workgroup total in *total.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < kBuildWaves ? s_wave[lane] : 0;
    int xs = w;
#pragma unroll
    for (int o = 1; o < kBuildWaves; o <<= 1) {
      const int y = __shfl_up(xs, o, 64);
      if (lane >= o) xs += y;
    }
    if (lane < kBuildWaves) s_wave[lane] = xs - w;
    if (lane == kBuildWaves - 1) s_wave[kBuildWaves] = xs;
  }
  __syncthreads();
  const int excl = s_wave[wave] + x - v;
  *total = s_wave[kBuildWaves];
  __syncthreads();
  return excl;
}

struct Segment {
  int32_t tok;   // first global token
  int32_t src;   // first emulated zigzag row
  int32_t len;   // tokens
  int32_t rank;  // zigzag (source) rank
};

__device__ __forceinline__ Segment make_segment(const int32_t* doc_start, const int32_t* doc_len, int k,
                                                int q, int cp, int share) {
  const int32_t a = doc_start[k];
  const int32_t c = doc_len[k] / (2 * cp);
  const bool back = q >= cp;
  Segment s;
  s.rank = back ? 2 * cp - 1 - q : q;
  s.tok = a + q * c;
  s.src = s.rank * share + a / cp + (back ? c : 0);
  s.len = c;
  return s;
}

// Segment j in zigzag-row order: rank-major, then document, then front/back.
__device__ __forceinline__ Segment segment_src_order(const int32_t* ds, const int32_t* dl, int64_t j, int n_docs,
                                                     int cp, int share) {
  const int r = static_cast<int>(j / (2 * n_docs));
  const int rem = static_cast<int>(j % (2 * n_docs));
  const int k = rem >> 1;
  const int q = (rem & 1) ? 2 * cp - 1 - r : r;
  return make_segment(ds, dl, k, q, cp, share);
}

// Segment j in token order: document-major, then chunk.
__device__ __forceinline__ Segment segment_tok_order(const int32_t* ds, const int32_t* dl, int64_t j, int cp,
                                                     int share) {
  const int k = static_cast<int>(j / (2 * cp));
  const int q = static_cast<int>(j % (2 * cp));
  return make_segment(ds, dl, k, q, cp, share);
}

__global__ __launch_bounds__(kBuildThreads) void route_build_kernel(const int32_t* __restrict__ cu, int32_t n_slots,
                                                                    int32_t cp, int32_t total, RouteDev ws) {
  __shared__ int s_wave[kBuildWaves + 1];
  __shared__ int s_sev;
  const int tid = threadIdx.x;

  // ---- 1. validate (precedence: start, monotone, total, divisibility) ----
  if (tid == 0) s_sev = 0;
  for (int i = tid; i < cp * cp; i += kBuildThreads)
    __hip_atomic_store(&ws.split[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wg_sync_global();
  int sev = 0;
  if (tid == 0) {
    if (cu[0] != 0) sev = kSevStart;
    if (cu[n_slots] != total) sev = max(sev, kSevTotal);
  }
  const int64_t two_cp = 2 * static_cast<int64_t>(cp);
  for (int i = tid; i < n_slots; i += kBuildThreads) {
    const int64_t a = cu[i], b = cu[i + 1];
    if (b < a) sev = max(sev, kSevMonotone);
    else if ((b - a) % two_cp != 0) sev = max(sev, kSevDivisible);
  }
  if (sev) atomicMax(&s_sev, sev);
  __syncthreads();
  if (s_sev) {
    if (tid == 0) {
      ws.hdr[kHdrRunsSrc] = 0;
      ws.hdr[kHdrRunsDst] = 0;
      ws.hdr[kHdrDocs] = 0;
      ws.hdr[kHdrCp] = cp;
      ws.hdr[kHdrTotal] = total;
      ws.hdr[kHdrStatus] = severity_to_code(s_sev);
    }
    return;
  }

  // ---- 2. compact: drop empty slots (repeated boundaries) ----
  int n_docs = 0;
  for (int base = 0; base < n_slots; base += kBuildThreads) {
    const int i = base + tid;
    int32_t a = 0, len = 0;
    if (i < n_slots) {
      a = cu[i];
      len = cu[i + 1] - a;
    }
    int sum;
    const int off = block_exclusive_scan(len > 0 ? 1 : 0, s_wave, &sum);
    if (len > 0) {
      ws.doc_start[n_docs + off] = a;
      ws.doc_len[n_docs + off] = len;
    }
    n_docs += sum;
  }
  wg_sync_global();

  const int share = total / cp;  // T/cp rows per rank (T is a multiple of 2*cp here)
  const int64_t n_seg = two_cp * n_docs;
  bool overflow = false;

  // ---- 3. runs in zigzag-row order, plus the split matrix ----
  int n_src = 0;
  for (int64_t base = 0; base < n_seg; base += kBuildThreads) {
    const int64_t j = base + tid;
    int count = 0, merge = 0, first_d = 0, pieces = 0;
    Segment s{};
    if (j < n_seg) {
      s = segment_src_order(ws.doc_start, ws.doc_len, j, n_docs, cp, share);
      first_d = s.tok / share;
      pieces = (s.tok + s.len - 1) / share - first_d + 1;
      if (s.src % share != 0 && s.tok % share != 0) {
        const Segment p = segment_src_order(ws.doc_start, ws.doc_len, j - 1, n_docs, cp, share);
        merge = (p.tok + p.len == s.tok) ? 1 : 0;
      }
      count = pieces - merge;
    }
    int sum;
    const int off = block_exclusive_scan(count, s_wave, &sum);
    if (j < n_seg) {
      for (int p = 0; p < pieces; ++p) {
        const int32_t ptok = p == 0 ? s.tok : (first_d + p) * share;
        const int32_t pend = min(s.tok + s.len, (first_d + p + 1) * share);
        atomicAdd(&ws.split[s.rank * cp + first_d + p], pend - ptok);
        if (p >= merge) {
          const int64_t slot = static_cast<int64_t>(n_src) + off + p - merge;
          if (slot < ws.run_cap) ws.runs_src[slot] = RunPair{s.src + (ptok - s.tok), ptok};
          else overflow = true;
        }
      }
    }
    n_src += sum;
  }

  // ---- 4. the same runs in token order ----
  int n_dst = 0;
  for (int64_t base = 0; base < n_seg; base += kBuildThreads) {
    const int64_t j = base + tid;
    int count = 0, merge = 0, first_d = 0, pieces = 0;
    Segment s{};
    if (j < n_seg) {
      s = segment_tok_order(ws.doc_start, ws.doc_len, j, cp, share);
      first_d = s.tok / share;
      pieces = (s.tok + s.len - 1) / share - first_d + 1;
      if (j > 0 && s.src % share != 0 && s.tok % share != 0) {
        const Segment p = segment_tok_order(ws.doc_start, ws.doc_len, j - 1, cp, share);
        merge = (p.src + p.len == s.src) ? 1 : 0;
      }
      count = pieces - merge;
    }
    int sum;
    const int off = block_exclusive_scan(count, s_wave, &sum);
    if (j < n_seg) {
      for (int p = merge; p < pieces; ++p) {
        const int32_t ptok = p == 0 ? s.tok : (first_d + p) * share;
        const int64_t slot = static_cast<int64_t>(n_dst) + off + p - merge;
        if (slot < ws.run_cap) ws.runs_dst[slot] = RunPair{ptok, s.src + (ptok - s.tok)};
        else overflow = true;
      }
    }
    n_dst += sum;
  }
  wg_sync_global();

  // ---- 5. integrity: same run count both ways; each rank sends and receives T/cp ----
  if (tid == 0) s_sev = 0;
  __syncthreads();
  bool bad = overflow || n_src != n_dst;
  for (int i = tid; i < cp; i += kBuildThreads) {
    int64_t row = 0, col = 0;
    for (int d = 0; d < cp; ++d) {
      row += __hip_atomic_load(&ws.split[i * cp + d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      col += __hip_atomic_load(&ws.split[d * cp + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (row != share || col != share) bad = true;
  }
  if (bad) atomicMax(&s_sev, 1);
  __syncthreads();
  if (tid == 0) {
    ws.hdr[kHdrRunsSrc] = n_src;
    ws.hdr[kHdrRunsDst] = n_dst;
    ws.hdr[kHdrDocs] = n_docs;
    ws.hdr[kHdrCp] = cp;
    ws.hdr[kHdrTotal] = total;
    ws.hdr[kHdrStatus] = s_sev ? THD_ERR_INTEGRITY : THD_OK;
  }
}

// Largest i in [0, n) with runs[i].out <= row (runs[0].out == 0 <= row).
__device__ __forceinline__ int32_t last_run_at_or_before(const RunPair* runs, int32_t n, int32_t row) {
  int32_t lo = 0, hi = n;  // runs[lo].out <= row, and runs[hi].out > row or hi == n
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (runs[mid].out <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ DirEntry dir_entry(const RunPair* runs, int32_t n, int32_t row, int32_t total) {
  const int32_t k = last_run_at_or_before(runs, n, row);
  const RunPair r = runs[k];
  DirEntry e;
  e.in = r.in + (row - r.out);
  e.run_end = k + 1 < n ? runs[k + 1].out : total;
  e.run = k;
  e.pad = 0;
  return e;
}

__global__ __launch_bounds__(256) void route_index_kernel(RouteDev ws, int32_t n_blocks, int32_t total) {
  if (ws.hdr[kHdrStatus] != THD_OK) return;
  const int32_t b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const int32_t row = b << kDirShift;
  ws.dir_src[b] = dir_entry(ws.runs_src, ws.hdr[kHdrRunsSrc], row, total);
  ws.dir_dst[b] = dir_entry(ws.runs_dst, ws.hdr[kHdrRunsDst], row, total);
}

}  // namespace

hipError_t launch_route_build(const int32_t* cu, int32_t n_slots, int32_t cp, int32_t total, const RouteDev& ws,
                              hipStream_t stream) {
  hipLaunchKernelGGL(route_build_kernel, dim3(1), dim3(kBuildThreads), 0, stream, cu, n_slots, cp, total, ws);
  return hipGetLastError();
}

hipError_t launch_route_index(const RouteDev& ws, int32_t total, hipStream_t stream) {
  const int32_t n_blocks = (total + kDirBlock - 1) / kDirBlock;
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(route_index_kernel, dim3((n_blocks + 255) / 256), dim3(256), 0, stream, ws, n_blocks, total);
  return hipGetLastError();
}

}  // namespace thdcp
