// Packing on the device: [batch, seq] token rows with PAD and EOD tokens ->
// one padded THD stream plus its real and padded boundary lists.
//
// Page "Packed Sequence 与上下文并行", §2.2 steps (1)-(3) and the worked
// example of §3.1-§3.4:
//  (1) in each row the valid part ends after the last non-PAD token; every
//      EOD inside it closes a document (the EOD is the document's last
//      token) and whatever follows the last EOD is one more document;
//  (2) each document is padded at its end to a multiple of `align`;
//  (3) the documents are laid end to end at their padded offsets, pads get
//      `pad_value`.
// The pages do (1) with a scan over segment ids and a bincount, (2) and (3)
// with host-side offset arithmetic.  Here three stream-ordered kernels do it
// with no host round trip, into a fixed token budget `capacity` with a fixed
// number of document slots `max_docs`: the space after the last document is
// one trailing pad-only slot and unused slots repeat the last boundary.  So
// every shape the route build, the swaps and the roll need is known on the
// host before the data is.
#include "thd_device.h"
#include "thd_internal.h"

namespace thdcp {
namespace {

constexpr int kPackThreads = 1024;
constexpr int kPackWaves = kPackThreads / 64;

// Rows: valid end, document ends (exclusive, row coordinates) and the row's
// padded token count.
__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(const int64_t* __restrict__ tokens, int32_t seq,
                                                                 int64_t pad_id, int64_t eod_id, int32_t align,
                                                                 PackWs ws) {
  __shared__ int s_wave[kPackWaves + 1];
  __shared__ int64_t s_wave64[kPackWaves + 1];
  __shared__ int s_valid, s_cnt;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t* row = tokens + b * seq;
  int32_t* ends = ws.ends + b * seq;

  if (tid == 0) s_valid = 0;
  __syncthreads();
  int last = 0;
  for (int32_t s = tid; s < seq; s += kPackThreads)
    if (row[s] != pad_id) last = max(last, s + 1);
  if (last) atomicMax(&s_valid, last);
  __syncthreads();
  const int32_t valid_end = s_valid;

  int32_t cnt = 0;
  for (int32_t base = 0; base < valid_end; base += kPackThreads) {
    const int32_t s = base + tid;
    const bool eod = s < valid_end && row[s] == eod_id;
    int sum;
    const int off = block_exclusive_scan<kPackThreads, int>(eod ? 1 : 0, s_wave, &sum);
    if (eod) ends[cnt + off] = s + 1;
    cnt += sum;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int32_t last_end = cnt ? ends[cnt - 1] : 0;
    if (valid_end > last_end) ends[cnt++] = valid_end;  // the document after the last EOD
    s_cnt = cnt;
  }
  __threadfence();
  __syncthreads();
  cnt = s_cnt;

  int64_t padded = 0;
  for (int32_t k = tid; k < cnt; k += kPackThreads) {
    const int32_t len = ends[k] - (k ? ends[k - 1] : 0);
    padded += len + (align - len % align) % align;
  }
  int64_t row_padded;
  block_exclusive_scan<kPackThreads, int64_t>(padded, s_wave64, &row_padded);
  if (tid == 0) {
    ws.row_valid[b] = valid_end;
    ws.row_docs[b] = cnt;
    ws.row_padded[b] = row_padded;
  }
}

// Prefix sums over rows, the budget checks and the boundary tails.
__global__ __launch_bounds__(kPackThreads) void pack_meta_kernel(int32_t batch, int32_t max_docs, int32_t capacity,
                                                                 PackWs ws, int32_t* __restrict__ cu_real,
                                                                 int32_t* __restrict__ cu_pad,
                                                                 int32_t* __restrict__ status) {
  __shared__ int64_t s_wave[kPackWaves + 1];
  const int tid = threadIdx.x;
  int64_t docs = 0, real = 0, padded = 0;
  for (int32_t base = 0; base < batch; base += kPackThreads) {
    const int32_t b = base + tid;
    const bool in = b < batch;
    int64_t sd, sr, sp;
    const int64_t od = block_exclusive_scan<kPackThreads, int64_t>(in ? ws.row_docs[b] : 0, s_wave, &sd);
    const int64_t orl = block_exclusive_scan<kPackThreads, int64_t>(in ? ws.row_valid[b] : 0, s_wave, &sr);
    const int64_t op = block_exclusive_scan<kPackThreads, int64_t>(in ? ws.row_padded[b] : 0, s_wave, &sp);
    if (in) {
      ws.row_doc_off[b] = docs + od;
      ws.row_real_off[b] = real + orl;
      ws.row_pack_off[b] = padded + op;
    }
    docs += sd;
    real += sr;
    padded += sp;
  }
  const int32_t code = docs > max_docs ? THD_ERR_PACK_DOCS : (padded > capacity ? THD_ERR_PACK_CAPACITY : THD_OK);
  if (tid == 0) {
    ws.hdr[0] = code;
    ws.hdr[1] = static_cast<int32_t>(min(docs, static_cast<int64_t>(INT32_MAX)));
    ws.hdr[2] = static_cast<int32_t>(min(padded, static_cast<int64_t>(INT32_MAX)));
    if (status) *status = code;
  }
  if (code != THD_OK) return;
  if (tid == 0) {
    cu_real[0] = 0;
    cu_pad[0] = 0;
  }
  // trailing pad slot (ends at the budget, no real tokens) and empty slots
  for (int64_t k = docs + 1 + tid; k <= static_cast<int64_t>(max_docs) + 1; k += kPackThreads) {
    cu_real[k] = static_cast<int32_t>(real);
    cu_pad[k] = capacity;
  }
}

// Per row: the documents' boundaries, their tokens and their pads; all
// workgroups together fill the trailing pad slot.
__global__ __launch_bounds__(kPackThreads) void pack_write_kernel(const int64_t* __restrict__ tokens, int32_t batch,
                                                                  int32_t seq, int32_t align, int64_t pad_value,
                                                                  int32_t capacity, PackWs ws,
                                                                  int64_t* __restrict__ packed,
                                                                  int32_t* __restrict__ cu_real,
                                                                  int32_t* __restrict__ cu_pad) {
  __shared__ int64_t s_wave[kPackWaves + 1];
  if (ws.hdr[0] != THD_OK) return;  // over budget: nothing is written
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  if (b < batch) {
    const int64_t* row = tokens + b * seq;
    const int32_t* ends = ws.ends + b * seq;
    const int32_t cnt = ws.row_docs[b];
    const int32_t valid_end = ws.row_valid[b];
    const int64_t doc_off = ws.row_doc_off[b];
    const int64_t real_off = ws.row_real_off[b];
    const int64_t pack_off = ws.row_pack_off[b];

    int64_t carry = pack_off;
    for (int32_t base = 0; base < cnt; base += kPackThreads) {
      const int32_t k = base + tid;
      int64_t plen = 0;
      if (k < cnt) {
        const int32_t len = ends[k] - (k ? ends[k - 1] : 0);
        plen = len + (align - len % align) % align;
      }
      int64_t sum;
      const int64_t off = block_exclusive_scan<kPackThreads, int64_t>(plen, s_wave, &sum);
      if (k < cnt) {
        cu_pad[doc_off + k + 1] = static_cast<int32_t>(carry + off + plen);
        cu_real[doc_off + k + 1] = static_cast<int32_t>(real_off + ends[k]);
      }
      carry += sum;
    }
    __threadfence();
    __syncthreads();  // this row's boundaries are read back below

    for (int32_t s = tid; s < valid_end; s += kPackThreads) {
      int32_t lo = 0, hi = cnt - 1;  // document k: the first with ends[k] > s
      while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (ends[mid] > s) hi = mid;
        else lo = mid + 1;
      }
      const int32_t start = lo ? ends[lo - 1] : 0;
      const int64_t base_pos = lo ? static_cast<int64_t>(cu_pad[doc_off + lo]) : pack_off;
      packed[base_pos + (s - start)] = row[s];
    }
    for (int32_t k = tid; k < cnt; k += kPackThreads) {
      const int32_t len = ends[k] - (k ? ends[k - 1] : 0);
      const int64_t begin = (k ? static_cast<int64_t>(cu_pad[doc_off + k]) : pack_off) + len;
      const int64_t end = cu_pad[doc_off + k + 1];
      for (int64_t p = begin; p < end; ++p) packed[p] = pad_value;
    }
  }
  const int64_t used = ws.hdr[2];
  for (int64_t i = used + static_cast<int64_t>(blockIdx.x) * kPackThreads + tid; i < capacity;
       i += static_cast<int64_t>(gridDim.x) * kPackThreads)
    packed[i] = pad_value;
}

}  // namespace

hipError_t launch_pack(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id,
                       int32_t align, int32_t capacity, int32_t max_docs, int64_t pad_value, const PackWs& ws,
                       int64_t* packed, int32_t* cu_real, int32_t* cu_pad, int32_t* status, hipStream_t stream) {
  if (batch > 0) {
    hipLaunchKernelGGL(pack_rows_kernel, dim3(batch), dim3(kPackThreads), 0, stream, tokens, seq, pad_id, eod_id,
                       align, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pack_meta_kernel, dim3(1), dim3(kPackThreads), 0, stream, batch, max_docs, capacity, ws, cu_real,
                     cu_pad, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t grid = batch > 0 ? batch : 1;
  hipLaunchKernelGGL(pack_write_kernel, dim3(grid), dim3(kPackThreads), 0, stream, tokens, batch, seq, align,
                     pad_value, capacity, ws, packed, cu_real, cu_pad);
  return hipGetLastError();
}

}  // namespace thdcp
