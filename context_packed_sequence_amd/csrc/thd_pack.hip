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
//
// Work decomposition: every row is cut into chunks of kChunk tokens and each
// chunk is one workgroup, so a batch of a few long rows still fills the chip.
//  * chunk pass: per chunk, the last non-PAD position, the number of EODs, the
//    first and last EOD, and the padded lengths of the documents that start
//    and end inside the chunk;
//  * scan pass (one workgroup): scans over all chunks in batch order give
//    each chunk the end of the last document closed before it, its first
//    document index and the packed position of the document it starts in;
//    the row sums give the trailing document of each row, and the totals
//    give the budget checks;
//  * write pass: per chunk, the tokens go to their packed positions, each
//    document end writes its two boundaries, and the chunk's pads are spread
//    over all its threads.
#include "thd_device.h"
#include "thd_internal.h"

namespace thdcp {
namespace {

constexpr int kChunk = 1024;          // tokens per chunk (one workgroup)
constexpr int kChunkThreads = 256;
constexpr int kPer = kChunk / kChunkThreads;  // consecutive tokens per thread
constexpr int kScanThreads = 1024;
constexpr int kFusedChunks = 256;  // up to this many chunks (one scan pass) each write workgroup runs the scan itself

// Length of a document of `len` tokens once padded to a multiple of align.
__device__ __forceinline__ int64_t padded_len(int32_t len, int32_t align) {
  const int32_t r = len % align;
  return static_cast<int64_t>(len) + (r ? align - r : 0);
}

// Chunk pass.
__global__ __launch_bounds__(kChunkThreads) void pack_chunks_kernel(const int64_t* __restrict__ tokens, int32_t seq,
                                                                    int32_t n_ch, int64_t pad_id, int64_t eod_id,
                                                                    int32_t align, PackWs ws) {
  __shared__ int64_t s_scan[3 * (kChunkThreads / 64 + 1)];
  const int tid = threadIdx.x;
  const int32_t c = blockIdx.x;
  const int32_t b = c / n_ch;
  const int32_t s0 = (c - b * n_ch) * kChunk + tid * kPer;
  const int64_t* row = tokens + static_cast<int64_t>(b) * seq;

  int32_t lnp = 0, ne = 0, fe = INT32_MAX, le = 0;
  bool eod[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int32_t s = s0 + i;
    const int64_t v = s < seq ? row[s] : pad_id;
    eod[i] = s < seq && v == eod_id;
    if (v != pad_id) lnp = s + 1;
    if (eod[i]) {
      ++ne;
      fe = min(fe, s + 1);
      le = s + 1;
    }
  }
  // maxima: the last EOD before this thread inside the chunk (0: none), and
  // the chunk's last non-PAD and (negated) first EOD
  const int64_t mv[3] = {le, lnp, -static_cast<int64_t>(fe)};
  int64_t mx[3], mt[3];
  block_exclusive_multi<kChunkThreads, 3, true>(mv, -static_cast<int64_t>(INT32_MAX), s_scan, mx, mt);
  int64_t ps = 0;  // padded lengths of documents with both ends in the chunk
  int32_t last = static_cast<int32_t>(max(mx[0], int64_t(0)));
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (eod[i]) {
      if (last > 0) ps += padded_len(s0 + i + 1 - last, align);
      last = s0 + i + 1;
    }
  }
  const int64_t sv[2] = {ne, ps};
  int64_t sx[2], st[2];
  block_exclusive_multi<kChunkThreads, 2, false>(sv, 0, s_scan, sx, st);
  if (tid == 0) {
    ws.ch_lnp[c] = static_cast<int32_t>(mt[1]);
    ws.ch_ne[c] = static_cast<int32_t>(st[0]);
    ws.ch_fe[c] = st[0] ? static_cast<int32_t>(-mt[2]) : 0;
    ws.ch_le[c] = static_cast<int32_t>(mt[0]);
    ws.ch_ps[c] = st[1];
  }
}

// What the scan over all chunks gives one chunk and its row.
struct ChunkPlace {
  int32_t prev;        // end of the last document of the row closed before the chunk
  int32_t valid_end;   // the row's valid end
  int64_t doc_base;    // index of the first document that ends in or after the chunk
  int64_t pack_base;   // packed position of the document holding the chunk's first token
  int64_t real_off;    // valid tokens of the earlier rows
};

struct PackTotals {
  int64_t docs, padded, real;
};

// Scan over all chunks in batch order, by one workgroup of kThreads.  Row
// boundaries are handled without segmented scans: a position p of row b is
// keyed b * (seq + 1) + p, so a running maximum never carries a value from an
// earlier row past the row's own base key.  With `store`, every chunk's and
// row's results go to the workspace; with want >= 0, those of chunk `want`
// and its row go to *place (LDS).  Every thread gets the totals.
template <int kThreads>
__device__ PackTotals scan_chunks(int32_t n_total, int32_t seq, int32_t n_ch, int32_t align, const PackWs& ws,
                                  int64_t* s_scan, bool store, int32_t want, ChunkPlace* place) {
  const int tid = threadIdx.x;
  const int64_t stride = static_cast<int64_t>(seq) + 1;
  const int32_t want_row = want >= 0 ? want / n_ch : -1;
  int64_t carry_eod = 0, carry_np = 0;            // running maxima of the keyed positions
  int64_t carry_d = 0, carry_p = 0, carry_r = 0;  // running sums: documents, padded, real
  for (int32_t base = 0; base < n_total; base += kThreads) {
    const int32_t c = base + tid;
    const bool in = c < n_total;
    const int32_t b = in ? c / n_ch : 0;
    const bool row_last = in && c - b * n_ch == n_ch - 1;
    int32_t ne = 0, le = 0, lnp = 0, fe = 0;
    int64_t ps = 0;
    if (in) {
      ne = ws.ch_ne[c];
      le = ws.ch_le[c];
      lnp = ws.ch_lnp[c];
      fe = ws.ch_fe[c];
      ps = ws.ch_ps[c];
    }
    const int64_t key0 = b * stride;
    const int64_t mv[2] = {in ? key0 + le : 0, in ? key0 + lnp : 0};
    int64_t mx[2], mt[2];
    block_exclusive_multi<kThreads, 2, true>(mv, 0, s_scan, mx, mt);
    const int64_t ex_eod = max(mx[0], carry_eod), ex_np = max(mx[1], carry_np);
    carry_eod = max(carry_eod, mt[0]);
    carry_np = max(carry_np, mt[1]);

    // end of the last document closed before this chunk (row coordinates)
    const int32_t prev_end = static_cast<int32_t>(max(ex_eod, key0) - key0);
    int64_t d = ne, p = 0, r = 0;
    int32_t valid_end = 0;
    if (ne) p = padded_len(fe - prev_end, align) + ps;
    if (row_last) {
      valid_end = static_cast<int32_t>(max(max(ex_np, mv[1]), key0) - key0);
      const int32_t last_eod = static_cast<int32_t>(max(max(ex_eod, mv[0]), key0) - key0);
      if (valid_end > last_eod) {  // the document after the row's last EOD
        d += 1;
        p += padded_len(valid_end - last_eod, align);
      }
      r = valid_end;
    }
    const int64_t sv[3] = {d, p, r};
    int64_t sx[3], st[3];
    block_exclusive_multi<kThreads, 3, false>(sv, 0, s_scan, sx, st);
    if (in) {
      if (store) {
        ws.ch_prev[c] = prev_end;
        ws.ch_doc_base[c] = carry_d + sx[0];
        ws.ch_pack_base[c] = carry_p + sx[1];
        if (row_last) {
          ws.row_valid[b] = valid_end;
          ws.row_real_off[b] = carry_r + sx[2];  // real tokens of the earlier rows
        }
      }
      if (c == want) {
        place->prev = prev_end;
        place->doc_base = carry_d + sx[0];
        place->pack_base = carry_p + sx[1];
      }
      if (row_last && b == want_row) {
        place->valid_end = valid_end;
        place->real_off = carry_r + sx[2];
      }
    }
    carry_d += st[0];
    carry_p += st[1];
    carry_r += st[2];
  }
  return PackTotals{carry_d, carry_p, carry_r};
}

// Status, header and the boundary lists' tail (the trailing pad slot, which
// ends at the budget with no real tokens, and the empty slots), by one
// workgroup.  Returns the status.
template <int kThreads>
__device__ int32_t pack_finish(const PackTotals& t, int32_t max_docs, int32_t capacity, const PackWs& ws,
                               int32_t* cu_real, int32_t* cu_pad, int32_t* status) {
  const int tid = threadIdx.x;
  const int32_t code =
      t.docs > max_docs ? THD_ERR_PACK_DOCS : (t.padded > capacity ? THD_ERR_PACK_CAPACITY : THD_OK);
  if (tid == 0) {
    ws.hdr[0] = code;
    ws.hdr[1] = static_cast<int32_t>(min(t.docs, static_cast<int64_t>(INT32_MAX)));
    ws.hdr[2] = static_cast<int32_t>(min(t.padded, static_cast<int64_t>(INT32_MAX)));
    if (status) *status = code;
  }
  if (code != THD_OK) return code;
  if (tid == 0) {
    cu_real[0] = 0;
    cu_pad[0] = 0;
  }
  for (int64_t k = t.docs + 1 + tid; k <= static_cast<int64_t>(max_docs) + 1; k += kThreads) {
    cu_real[k] = static_cast<int32_t>(t.real);
    cu_pad[k] = capacity;
  }
  return code;
}

// Scan pass for batches of many chunks: one workgroup.
__global__ __launch_bounds__(kScanThreads) void pack_scan_kernel(int32_t n_total, int32_t seq, int32_t n_ch,
                                                                 int32_t align, int32_t max_docs, int32_t capacity,
                                                                 PackWs ws, int32_t* __restrict__ cu_real,
                                                                 int32_t* __restrict__ cu_pad,
                                                                 int32_t* __restrict__ status) {
  __shared__ int64_t s_scan[3 * (kScanThreads / 64 + 1)];
  const PackTotals t = scan_chunks<kScanThreads>(n_total, seq, n_ch, align, ws, s_scan, true, -1, nullptr);
  pack_finish<kScanThreads>(t, max_docs, capacity, ws, cu_real, cu_pad, status);
}

struct PadRun {
  int64_t start;  // packed position of the run's first pad
  int64_t first;  // index of that pad among the chunk's pads
};

// Write pass: one workgroup per chunk, then every workgroup helps fill the
// budget's tail.  kFused (batches of at most kFusedChunks chunks): every
// workgroup first runs the scan over all chunks itself, keeping only its own
// chunk's results, and workgroup 0 writes the status and the lists' tail, so
// the separate scan launch is not needed.
template <bool kFused>
__global__ __launch_bounds__(kChunkThreads) void pack_write_kernel(const int64_t* __restrict__ tokens, int32_t seq,
                                                                   int32_t n_ch, int32_t n_chunks, int64_t eod_id,
                                                                   int32_t align, int64_t pad_value,
                                                                   int32_t capacity, int32_t max_docs, PackWs ws,
                                                                   int64_t* __restrict__ packed,
                                                                   int32_t* __restrict__ cu_real,
                                                                   int32_t* __restrict__ cu_pad,
                                                                   int32_t* __restrict__ status) {
  __shared__ int64_t s_scan[3 * (kChunkThreads / 64 + 1)];
  __shared__ PadRun s_pads[kChunk];
  __shared__ ChunkPlace s_place;
  const int tid = threadIdx.x;
  const int32_t c = blockIdx.x;
  // The chunk's tokens do not depend on the scan (only the row's valid end,
  // applied below, does): they are read first, in the same memory round trip
  // as the scan's reads.
  const int32_t b = c < n_chunks ? c / n_ch : 0;
  const int32_t chunk_start = (c - b * n_ch) * kChunk;
  const int32_t s0 = chunk_start + tid * kPer;
  const int64_t* row = tokens + static_cast<int64_t>(b) * seq;
  int64_t v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) v[i] = c < n_chunks && s0 + i < seq ? row[s0 + i] : 0;
  int64_t used;
  if constexpr (kFused) {
    const PackTotals t =
        scan_chunks<kChunkThreads>(n_chunks, seq, n_ch, align, ws, s_scan, false, c < n_chunks ? c : -1, &s_place);
    int32_t code;
    if (c == 0) code = pack_finish<kChunkThreads>(t, max_docs, capacity, ws, cu_real, cu_pad, status);
    else code = t.docs > max_docs || t.padded > capacity ? THD_ERR_PACK_DOCS : THD_OK;
    if (code != THD_OK) return;  // over budget: nothing is written
    used = t.padded;
    __syncthreads();  // s_place is complete
  } else {
    if (ws.hdr[0] != THD_OK) return;  // over budget: nothing is written
    used = ws.hdr[2];
    if (tid == 0 && c < n_chunks)
      s_place = ChunkPlace{ws.ch_prev[c], ws.row_valid[b], ws.ch_doc_base[c], ws.ch_pack_base[c],
                           ws.row_real_off[b]};
    __syncthreads();
  }
  if (c < n_chunks) {
    const int32_t valid_end = s_place.valid_end;
    if (chunk_start < valid_end) {  // uniform per workgroup
      bool end[kPer];
      int32_t le = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int32_t s = s0 + i;
        end[i] = s < valid_end && (v[i] == eod_id || s + 1 == valid_end);
        if (end[i]) le = s + 1;
      }
      const int64_t mv[1] = {le};
      int64_t mx[1], mt[1];
      block_exclusive_multi<kChunkThreads, 1, true>(mv, 0, s_scan, mx, mt);
      const int32_t start0 = max(static_cast<int32_t>(mx[0]), s_place.prev);
      int64_t plen_sum = 0, pad_sum = 0, n_end = 0;
      int32_t st = start0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (end[i]) {
          const int32_t len = s0 + i + 1 - st;
          const int64_t pl = padded_len(len, align);
          plen_sum += pl;
          pad_sum += pl - len;
          ++n_end;
          st = s0 + i + 1;
        }
      }
      const int64_t sv[3] = {plen_sum, pad_sum, n_end};
      int64_t sx[3], stot[3];
      block_exclusive_multi<kChunkThreads, 3, false>(sv, 0, s_scan, sx, stot);
      const int64_t pl_off = sx[0], pad_off = sx[1], pad_total = stot[1];
      // a chunk holds at most kChunk document ends
      const int32_t end_off = static_cast<int32_t>(sx[2]);
      const int32_t end_total = static_cast<int32_t>(min(stot[2], static_cast<int64_t>(kChunk)));

      const int64_t real_off = s_place.real_off;
      int64_t pos = s_place.pack_base + pl_off;  // packed start of the current document
      int64_t k = s_place.doc_base + end_off;    // its index
      int64_t pads_seen = pad_off;
      int32_t slot = end_off;
      st = start0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int32_t s = s0 + i;
        // the scans keep every position inside the budget and every document
        // inside the slots once the budget checks passed; the guards only
        // make that independent of the workspace's contents
        if (s < valid_end && pos + (s - st) < capacity) packed[pos + (s - st)] = v[i];
        if (end[i]) {
          const int32_t len = s + 1 - st;
          const int64_t pl = padded_len(len, align);
          if (k < max_docs) {
            cu_real[k + 1] = static_cast<int32_t>(real_off + s + 1);
            cu_pad[k + 1] = static_cast<int32_t>(pos + pl);
          }
          if (slot < kChunk) s_pads[slot] = PadRun{pos + len, pads_seen};
          pads_seen += pl - len;
          ++slot;
          ++k;
          pos += pl;
          st = s + 1;
        }
      }
      __syncthreads();
      // the chunk's pads, spread over every thread: pad q belongs to the last
      // document end whose first pad index is <= q
      for (int64_t q = tid; end_total > 0 && q < pad_total; q += kChunkThreads) {
        int32_t lo = 0, hi = end_total;
        while (hi - lo > 1) {
          const int32_t mid = (lo + hi) >> 1;
          if (s_pads[mid].first <= q) lo = mid;
          else hi = mid;
        }
        const int64_t at = s_pads[lo].start + (q - s_pads[lo].first);
        if (at < capacity) packed[at] = pad_value;
      }
    }
  }
  for (int64_t i = used + static_cast<int64_t>(blockIdx.x) * kChunkThreads + tid; i < capacity;
       i += static_cast<int64_t>(gridDim.x) * kChunkThreads)
    packed[i] = pad_value;
}

}  // namespace

int64_t pack_chunks(int32_t batch, int32_t seq) {
  const int64_t n_ch = (static_cast<int64_t>(seq) + kChunk - 1) / kChunk;
  return static_cast<int64_t>(batch) * n_ch;
}

hipError_t launch_pack(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id,
                       int32_t align, int32_t capacity, int32_t max_docs, int64_t pad_value, const PackWs& ws,
                       int64_t* packed, int32_t* cu_real, int32_t* cu_pad, int32_t* status, hipStream_t stream) {
  const int32_t n_ch = static_cast<int32_t>((static_cast<int64_t>(seq) + kChunk - 1) / kChunk);
  const int64_t n_chunks = pack_chunks(batch, seq);
  if (n_chunks > INT32_MAX) return hipErrorInvalidValue;
  if (n_chunks > 0) {
    hipLaunchKernelGGL(pack_chunks_kernel, dim3(static_cast<unsigned>(n_chunks)), dim3(kChunkThreads), 0, stream,
                       tokens, seq, n_ch, pad_id, eod_id, align, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int32_t n_ch_arg = n_ch > 0 ? n_ch : 1;
  const int64_t grid = n_chunks > 0 ? n_chunks : 1;
#define THD_PACK_WRITE(F)                                                                                           \
  hipLaunchKernelGGL((pack_write_kernel<F>), dim3(static_cast<unsigned>(grid)), dim3(kChunkThreads), 0, stream,     \
                     tokens, seq, n_ch_arg, static_cast<int32_t>(n_chunks), eod_id, align, pad_value, capacity,      \
                     max_docs, ws, packed, cu_real, cu_pad, status)
  if (n_chunks <= kFusedChunks) {
    THD_PACK_WRITE(true);
  } else {
    hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, static_cast<int32_t>(n_chunks), seq,
                       n_ch_arg, align, max_docs, capacity, ws, cu_real, cu_pad, status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    THD_PACK_WRITE(false);
  }
#undef THD_PACK_WRITE
  return hipGetLastError();
}

}  // namespace thdcp
