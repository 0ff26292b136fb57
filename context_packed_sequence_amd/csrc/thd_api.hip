// C ABI of libthdcp: host-side argument checks, the route object and
// stream-ordered launches.  See include/thd_cp.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "thd_cp_bench.h"
#include "thd_internal.h"

using thdcp::RouteDev;
using thdcp::RunPair;

struct thd_route {
  int device = -1;
  int32_t max_slots = 0;
  int32_t max_cp = 0;
  int64_t max_tokens = 0;
  int64_t run_cap = 0;
  int64_t dir_cap = 0;
  void* base = nullptr;
  RouteDev dev{};
  // shape of the last build (host-known, so no call ever needs a device read)
  int built = 0;
  int32_t cp = 0;
  int64_t total = 0;
  int32_t n_slots = 0;
  // launch-shape override of this route's swaps (thd_route_launch_shape)
  thdcp::SwapLaunch launch{0, 1, 0, 0};
};

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

bool on_route_device(const thd_route* r) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  return dev == r->device;
}

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  if (a_bytes <= 0 || b_bytes <= 0) return false;
  const auto x = reinterpret_cast<uintptr_t>(a);
  const auto y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uint64_t>(b_bytes) && y < x + static_cast<uint64_t>(a_bytes);
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Typical run length of the last build, in rows: its tokens over its 2 * cp
// zigzag segments per slot (empty slots counted, so never an overestimate of
// the average segment).  Chooses the swap path for one-unit rows.
int64_t typical_run_rows(const thd_route* r) {
  const int64_t segments = 2LL * r->cp * (r->n_slots > 0 ? r->n_slots : 1);
  return r->total / segments;
}

int check_roll_args(const int64_t* ids, const int32_t* cu_pad, int32_t n_slots, int64_t total, int32_t max_shift,
                    const int64_t* shifted, const uint8_t* mask, const int32_t* status) {
  if (!cu_pad || n_slots < 0 || total < 0 || total > INT32_MAX) return THD_ERR_ARG;
  if (max_shift < 1 || max_shift > THD_MAX_SHIFT) return THD_ERR_ARG;
  if (total > 0 && (!ids || !shifted || !mask)) return THD_ERR_ARG;
  const int64_t t = total;
  if (overlaps(shifted, t * max_shift * 8, ids, t * 8) || overlaps(mask, t * (max_shift + 1), ids, t * 8) ||
      overlaps(mask, t * (max_shift + 1), shifted, t * max_shift * 8))
    return THD_ERR_ALIAS;
  if (status && (overlaps(status, 4, shifted, t * max_shift * 8) || overlaps(status, 4, mask, t * (max_shift + 1))))
    return THD_ERR_ALIAS;
  return THD_OK;
}

}  // namespace

extern "C" {

const char* thd_strerror(int32_t code) {
  switch (code) {
    case THD_OK: return "ok";
    case THD_IDENTITY: return "identity route: nothing written, use the input";
    case THD_ERR_ARG: return "invalid argument";
    case THD_ERR_DIRECTION: return "invalid direction";
    case THD_ERR_NOT_BUILT: return "route was never built";
    case THD_ERR_ALIAS: return "input and output ranges overlap";
    case THD_ERR_CAPACITY: return "size exceeds the route's capacity";
    case THD_ERR_SHAPE: return "row count differs from the route's total tokens";
    case THD_ERR_HIP: return "HIP runtime error";
    case THD_ERR_DEVICE: return "current device is not the route's device";
    case THD_ERR_CU_START: return "cu_seqlens[0] is not 0";
    case THD_ERR_CU_MONOTONE: return "cu_seqlens decreases";
    case THD_ERR_CU_TOTAL: return "cu_seqlens[-1] differs from total tokens";
    case THD_ERR_CU_DIVISIBLE: return "a sequence length is not a multiple of 2*cp_size";
    case THD_ERR_REAL_GT_PADDED: return "a real sequence length exceeds its padded length";
    case THD_ERR_INTEGRITY: return "route integrity check failed";
    case THD_ERR_PACK_DOCS: return "more documents than document slots";
    case THD_ERR_PACK_CAPACITY: return "padded documents exceed the token budget";
    default: return "unknown code";
  }
}

int thd_route_create(int32_t max_slots, int32_t max_cp, int64_t max_tokens, thd_route** out) {
  if (!out) return THD_ERR_ARG;
  *out = nullptr;
  if (max_slots < 1 || max_cp < 1 || max_cp > THD_MAX_CP || max_tokens < 1 || max_tokens > INT32_MAX)
    return THD_ERR_ARG;
  thd_route* r = new (std::nothrow) thd_route();
  if (!r) return THD_ERR_ARG;
  if (hipGetDevice(&r->device) != hipSuccess) {
    delete r;
    return THD_ERR_HIP;
  }
  r->max_slots = max_slots;
  r->max_cp = max_cp;
  r->max_tokens = max_tokens;
  r->run_cap = 2LL * max_cp * max_slots + max_cp;
  r->dir_cap = (max_tokens + thdcp::kDirBlock - 1) / thdcp::kDirBlock + 1;

  int64_t off = 0;
  const int64_t o_hdr = off;       off = align_up(off + thdcp::kHdrWords * 4, 256);
  const int64_t o_src = off;       off = align_up(off + r->run_cap * 8, 256);
  const int64_t o_dst = off;       off = align_up(off + r->run_cap * 8, 256);
  const int64_t o_split = off;     off = align_up(off + static_cast<int64_t>(max_cp) * max_cp * 4, 256);
  const int64_t o_dsrc = off;      off = align_up(off + r->dir_cap * 16, 256);
  const int64_t o_ddst = off;      off = align_up(off + r->dir_cap * 16, 256);
  const int64_t o_docs = off;      off = align_up(off + 3 * static_cast<int64_t>(max_slots) * 4, 256);
  if (hipMalloc(&r->base, static_cast<size_t>(off)) != hipSuccess) {
    delete r;
    return THD_ERR_HIP;
  }
  char* b = static_cast<char*>(r->base);
  r->dev.hdr = reinterpret_cast<int32_t*>(b + o_hdr);
  r->dev.runs_src = reinterpret_cast<RunPair*>(b + o_src);
  r->dev.runs_dst = reinterpret_cast<RunPair*>(b + o_dst);
  r->dev.split = reinterpret_cast<int32_t*>(b + o_split);
  r->dev.dir_src = reinterpret_cast<thdcp::DirEntry*>(b + o_dsrc);
  r->dev.dir_dst = reinterpret_cast<thdcp::DirEntry*>(b + o_ddst);
  r->dev.docs = reinterpret_cast<int32_t*>(b + o_docs);
  r->dev.docs_cap = max_slots;
  r->dev.run_cap = r->run_cap;
  *out = r;
  return THD_OK;
}

void thd_route_destroy(thd_route* route) {
  if (!route) return;
  if (route->base) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != route->device) (void)hipSetDevice(route->device);
    (void)hipFree(route->base);
    if (prev >= 0 && prev != route->device) (void)hipSetDevice(prev);
  }
  delete route;
}

int thd_build_route(thd_route* route, const int32_t* cu_seqlens_padded, int32_t n_slots, int32_t cp_size,
                    int64_t total_tokens, void* stream) {
  if (!route || !cu_seqlens_padded || n_slots < 0 || cp_size < 1 || total_tokens < 0 || total_tokens > INT32_MAX)
    return THD_ERR_ARG;
  if (n_slots > route->max_slots || cp_size > route->max_cp || total_tokens > route->max_tokens)
    return THD_ERR_CAPACITY;
  if (!on_route_device(route)) return THD_ERR_DEVICE;
  route->built = 0;
  route->cp = cp_size;
  route->total = total_tokens;
  route->n_slots = n_slots;
  if (cp_size == 1) {  // identity; the boundaries are not read
    route->built = 1;
    return THD_OK;
  }
  hipStream_t s = as_stream(stream);
  if (thdcp::launch_route_build(cu_seqlens_padded, n_slots, cp_size, static_cast<int32_t>(total_tokens), route->dev,
                                s) != hipSuccess)
    return THD_ERR_HIP;
  route->built = 1;
  return THD_OK;
}

int thd_swap(const thd_route* route, int32_t direction, const void* in, void* out, int64_t rows, int64_t row_bytes,
             void* stream) {
  if (!route || rows < 0 || row_bytes < 1) return THD_ERR_ARG;
  if (direction != THD_ZIGZAG_TO_CONTIGUOUS && direction != THD_CONTIGUOUS_TO_ZIGZAG) return THD_ERR_DIRECTION;
  if (!route->built) return THD_ERR_NOT_BUILT;
  if (rows != route->total) return THD_ERR_SHAPE;
  if (route->cp == 1 || rows == 0) return THD_IDENTITY;
  if (!in || !out) return THD_ERR_ARG;
  if (row_bytes > INT64_MAX / rows) return THD_ERR_ARG;
  const int64_t bytes = rows * row_bytes;
  if (overlaps(in, bytes, out, bytes)) return THD_ERR_ALIAS;
  if (!on_route_device(route)) return THD_ERR_DEVICE;
  const bool z2c = direction == THD_ZIGZAG_TO_CONTIGUOUS;
  const RunPair* runs = z2c ? route->dev.runs_dst : route->dev.runs_src;
  const thdcp::DirEntry* dir = z2c ? route->dev.dir_dst : route->dev.dir_src;
  const int word = z2c ? thdcp::kHdrRunsDst : thdcp::kHdrRunsSrc;
  if (thdcp::launch_swap(route->dev.hdr, runs, word, dir, in, out, static_cast<int32_t>(rows), row_bytes,
                         typical_run_rows(route), route->launch, as_stream(stream)) != hipSuccess)
    return THD_ERR_HIP;
  return THD_OK;
}

int thd_copy(const void* in, void* out, int64_t bytes, void* stream) {
  if (bytes < 0) return THD_ERR_ARG;
  if (bytes == 0) return THD_OK;
  if (!in || !out) return THD_ERR_ARG;
  if (overlaps(in, bytes, out, bytes)) return THD_ERR_ALIAS;
  if (thdcp::launch_copy(in, out, bytes, as_stream(stream)) != hipSuccess) return THD_ERR_HIP;
  return THD_OK;
}

int thd_read_stream(const void* in, int64_t bytes, const void* key, uint32_t* count, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return THD_ERR_ARG;
  if (bytes == 0) return THD_OK;
  if (!in || !key || !count) return THD_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(in) & 15) || (reinterpret_cast<uintptr_t>(count) & 3)) return THD_ERR_ARG;
  if (overlaps(in, bytes, count, 4)) return THD_ERR_ALIAS;
  uint32_t k[4];
  std::memcpy(k, key, sizeof(k));
  if (thdcp::launch_read_stream(in, bytes, k, count, as_stream(stream)) != hipSuccess) return THD_ERR_HIP;
  return THD_OK;
}

int thd_write_stream(void* out, int64_t bytes, uint32_t seed, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return THD_ERR_ARG;
  if (bytes == 0) return THD_OK;
  if (!out || (reinterpret_cast<uintptr_t>(out) & 15)) return THD_ERR_ARG;
  if (thdcp::launch_write_stream(out, bytes, seed, as_stream(stream)) != hipSuccess) return THD_ERR_HIP;
  return THD_OK;
}

int thd_roll_labels(const int64_t* ids, const int32_t* cu_seqlens_padded, const int32_t* cu_seqlens, int32_t n_slots,
                    int64_t total_tokens, int32_t max_shift, int64_t fill, int64_t* shifted, uint8_t* mask,
                    int32_t* status, void* stream) {
  const int rc = check_roll_args(ids, cu_seqlens_padded, n_slots, total_tokens, max_shift, shifted, mask, status);
  if (rc != THD_OK) return rc;
  if (thdcp::launch_roll(ids, cu_seqlens_padded, cu_seqlens, n_slots, static_cast<int32_t>(total_tokens), max_shift,
                         fill, shifted, mask, status, nullptr, as_stream(stream)) != hipSuccess)
    return THD_ERR_HIP;
  return THD_OK;
}

int thd_roll_labels_zigzag(const thd_route* route, const int64_t* ids, const int32_t* cu_seqlens_padded,
                           const int32_t* cu_seqlens, int32_t n_slots, int64_t total_tokens, int32_t max_shift,
                           int64_t fill, int64_t* shifted, uint8_t* mask, int32_t* status, void* stream) {
  if (!route) return THD_ERR_ARG;
  if (!route->built) return THD_ERR_NOT_BUILT;
  if (total_tokens != route->total || n_slots != route->n_slots) return THD_ERR_SHAPE;
  if (route->cp == 1 || total_tokens == 0)
    return thd_roll_labels(ids, cu_seqlens_padded, cu_seqlens, n_slots, total_tokens, max_shift, fill, shifted, mask,
                           status, stream);
  const int rc = check_roll_args(ids, cu_seqlens_padded, n_slots, total_tokens, max_shift, shifted, mask, status);
  if (rc != THD_OK) return rc;
  if (!on_route_device(route)) return THD_ERR_DEVICE;
  const thdcp::RollRoute rt{route->dev.hdr, route->dev.runs_dst, route->dev.dir_dst};
  if (thdcp::launch_roll(ids, cu_seqlens_padded, cu_seqlens, n_slots, static_cast<int32_t>(total_tokens), max_shift,
                         fill, shifted, mask, status, &rt, as_stream(stream)) != hipSuccess)
    return THD_ERR_HIP;
  return THD_OK;
}

int thd_swap_batch(const thd_route* route, int32_t direction, int32_t n_tensors, const void* const* ins,
                   void* const* outs, const int64_t* row_bytes, int64_t rows, void* stream) {
  if (!route || rows < 0 || n_tensors < 1 || n_tensors > THD_MAX_BATCH || !ins || !outs || !row_bytes)
    return THD_ERR_ARG;
  if (direction != THD_ZIGZAG_TO_CONTIGUOUS && direction != THD_CONTIGUOUS_TO_ZIGZAG) return THD_ERR_DIRECTION;
  if (!route->built) return THD_ERR_NOT_BUILT;
  if (rows != route->total) return THD_ERR_SHAPE;
  for (int32_t i = 0; i < n_tensors; ++i)
    if (row_bytes[i] < 1 || (rows > 0 && row_bytes[i] > INT64_MAX / rows)) return THD_ERR_ARG;
  if (route->cp == 1 || rows == 0) return THD_IDENTITY;
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (!ins[i] || !outs[i]) return THD_ERR_ARG;
    const int64_t bi = rows * row_bytes[i];
    for (int32_t j = 0; j < n_tensors; ++j) {
      const int64_t bj = rows * row_bytes[j];
      if (overlaps(outs[i], bi, ins[j], bj)) return THD_ERR_ALIAS;
      if (j != i && overlaps(outs[i], bi, outs[j], bj)) return THD_ERR_ALIAS;
    }
  }
  if (!on_route_device(route)) return THD_ERR_DEVICE;
  const bool z2c = direction == THD_ZIGZAG_TO_CONTIGUOUS;
  const RunPair* runs = z2c ? route->dev.runs_dst : route->dev.runs_src;
  const thdcp::DirEntry* dir = z2c ? route->dev.dir_dst : route->dev.dir_src;
  const int word = z2c ? thdcp::kHdrRunsDst : thdcp::kHdrRunsSrc;
  if (thdcp::launch_swap_batch(route->dev.hdr, runs, word, dir, n_tensors, ins, outs, row_bytes,
                               static_cast<int32_t>(rows), typical_run_rows(route), as_stream(stream)) != hipSuccess)
    return THD_ERR_HIP;
  return THD_OK;
}

namespace {

struct PackLayout {
  int64_t hdr, ch_lnp, ch_ne, ch_fe, ch_le, ch_ps, ch_prev, ch_doc_base, ch_pack_base, row_valid, row_real_off, bytes;
};

PackLayout pack_layout(int32_t batch, int32_t seq) {
  const int64_t nc = thdcp::pack_chunks(batch, seq);
  PackLayout l{};
  int64_t off = 0;
  l.hdr = off;          off = align_up(off + 64, 256);
  l.ch_lnp = off;       off = align_up(off + nc * 4, 256);
  l.ch_ne = off;        off = align_up(off + nc * 4, 256);
  l.ch_fe = off;        off = align_up(off + nc * 4, 256);
  l.ch_le = off;        off = align_up(off + nc * 4, 256);
  l.ch_ps = off;        off = align_up(off + nc * 8, 256);
  l.ch_prev = off;      off = align_up(off + nc * 4, 256);
  l.ch_doc_base = off;  off = align_up(off + nc * 8, 256);
  l.ch_pack_base = off; off = align_up(off + nc * 8, 256);
  l.row_valid = off;    off = align_up(off + static_cast<int64_t>(batch) * 4, 256);
  l.row_real_off = off; off = align_up(off + static_cast<int64_t>(batch) * 8, 256);
  l.bytes = off;
  return l;
}

}  // namespace

// Device scratch of thd_pack_noalloc, in place of the caller's workspace: a
// file-scope array, one copy on every GPU the library runs on, held until
// the process ends.  In host code its name is only a host-side stand-in;
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[THD_PACK_STATIC_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on `device` (the current device), looked up on the
// first call for that device and kept.
int scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return THD_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return THD_ERR_HIP;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return THD_OK;
}

}  // namespace

int64_t thd_pack_workspace_bytes(int32_t batch, int32_t seq) {
  if (batch < 0 || seq < 0 || seq > THD_PACK_MAX_SEQ) return -1;
  return pack_layout(batch, seq).bytes;
}

int thd_pack(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id, int32_t align,
             int64_t capacity, int32_t max_docs, int64_t pad_value, void* workspace, int64_t workspace_bytes,
             int64_t* packed, int32_t* cu_seqlens, int32_t* cu_seqlens_padded, int32_t* status, void* stream) {
  if (batch < 0 || seq < 0 || seq > THD_PACK_MAX_SEQ || align < 1 || capacity < 0 || capacity > INT32_MAX || capacity % align != 0 ||
      max_docs < 0 || max_docs > INT32_MAX - 2 || pad_id == eod_id)
    return THD_ERR_ARG;
  const int64_t n_tok = static_cast<int64_t>(batch) * seq;
  const PackLayout l = pack_layout(batch, seq);
  if (!workspace || workspace_bytes < l.bytes || !cu_seqlens || !cu_seqlens_padded) return THD_ERR_ARG;
  if ((n_tok > 0 && !tokens) || (capacity > 0 && !packed)) return THD_ERR_ARG;
  const int64_t cu_bytes = (static_cast<int64_t>(max_docs) + 2) * 4;
  const struct {
    const void* p;
    int64_t n;
  } outs[] = {{packed, capacity * 8}, {cu_seqlens, cu_bytes}, {cu_seqlens_padded, cu_bytes}, {status, status ? 4 : 0},
              {workspace, l.bytes}};
  for (size_t i = 0; i < 5; ++i) {
    if (overlaps(outs[i].p, outs[i].n, tokens, n_tok * 8)) return THD_ERR_ALIAS;
    for (size_t j = i + 1; j < 5; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return THD_ERR_ALIAS;
  }
  char* w = static_cast<char*>(workspace);
  thdcp::PackWs ws;
  ws.hdr = reinterpret_cast<int32_t*>(w + l.hdr);
  ws.ch_lnp = reinterpret_cast<int32_t*>(w + l.ch_lnp);
  ws.ch_ne = reinterpret_cast<int32_t*>(w + l.ch_ne);
  ws.ch_fe = reinterpret_cast<int32_t*>(w + l.ch_fe);
  ws.ch_le = reinterpret_cast<int32_t*>(w + l.ch_le);
  ws.ch_ps = reinterpret_cast<int64_t*>(w + l.ch_ps);
  ws.ch_prev = reinterpret_cast<int32_t*>(w + l.ch_prev);
  ws.ch_doc_base = reinterpret_cast<int64_t*>(w + l.ch_doc_base);
  ws.ch_pack_base = reinterpret_cast<int64_t*>(w + l.ch_pack_base);
  ws.row_valid = reinterpret_cast<int32_t*>(w + l.row_valid);
  ws.row_real_off = reinterpret_cast<int64_t*>(w + l.row_real_off);
  if (thdcp::launch_pack(tokens, batch, seq, pad_id, eod_id, align, static_cast<int32_t>(capacity), max_docs,
                         pad_value, ws, packed, cu_seqlens, cu_seqlens_padded, status, as_stream(stream)) != hipSuccess)
    return THD_ERR_HIP;
  return THD_OK;
}

int thd_pack_noalloc(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id, int32_t align,
                     int64_t capacity, int32_t max_docs, int64_t pad_value, int64_t* packed, int32_t* cu_seqlens,
                     int32_t* cu_seqlens_padded, int32_t* status, void* stream) {
  if (batch < 0 || seq < 0 || seq > THD_PACK_MAX_SEQ) return THD_ERR_ARG;
  if (pack_layout(batch, seq).bytes > THD_PACK_STATIC_BYTES) return THD_ERR_CAPACITY;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return THD_ERR_HIP;
  void* ws = nullptr;
  const int rc = scratch_address(device, &ws);
  if (rc != THD_OK) return rc;
  // nothing in the scratch has to start at zero: every word a pack reads was
  // written earlier in the same call
  return thd_pack(tokens, batch, seq, pad_id, eod_id, align, capacity, max_docs, pad_value, ws,
                  THD_PACK_STATIC_BYTES, packed, cu_seqlens, cu_seqlens_padded, status, stream);
}

int thd_route_status(const thd_route* route, void* stream, int32_t* host_status) {
  if (!route || !host_status) return THD_ERR_ARG;
  if (!route->built) return THD_ERR_NOT_BUILT;
  if (route->cp == 1) {
    *host_status = THD_OK;
    return THD_OK;
  }
  if (!on_route_device(route)) return THD_ERR_DEVICE;
  int32_t v = 0;
  hipStream_t s = as_stream(stream);
  if (hipMemcpyAsync(&v, route->dev.hdr + thdcp::kHdrStatus, 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return THD_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return THD_ERR_HIP;
  *host_status = v;
  return THD_OK;
}

int thd_route_copy_out(const thd_route* route, void* stream, int32_t* host_n_runs, int32_t capacity,
                       int32_t* host_runs_by_src, int32_t* host_runs_by_dst, int32_t* host_split) {
  if (!route || !host_n_runs || capacity < 0) return THD_ERR_ARG;
  if (!route->built) return THD_ERR_NOT_BUILT;
  if (route->cp == 1) {
    *host_n_runs = 0;
    return THD_OK;
  }
  if (!on_route_device(route)) return THD_ERR_DEVICE;
  hipStream_t s = as_stream(stream);
  int32_t hdr[thdcp::kHdrWords];
  if (hipMemcpyAsync(hdr, route->dev.hdr, sizeof(hdr), hipMemcpyDeviceToHost, s) != hipSuccess) return THD_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return THD_ERR_HIP;
  const int32_t n = hdr[thdcp::kHdrStatus] == THD_OK ? hdr[thdcp::kHdrRunsSrc] : 0;
  if (n < 0 || n > route->run_cap) return THD_ERR_INTEGRITY;  // never after a good build
  *host_n_runs = n;
  if (n > capacity) return THD_ERR_CAPACITY;
  const int32_t cp = route->cp;
  const int64_t total = route->total;
  std::vector<RunPair> a(static_cast<size_t>(n)), b(static_cast<size_t>(n));
  if (n > 0) {
    if (hipMemcpyAsync(a.data(), route->dev.runs_src, n * sizeof(RunPair), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(b.data(), route->dev.runs_dst, n * sizeof(RunPair), hipMemcpyDeviceToHost, s) != hipSuccess)
      return THD_ERR_HIP;
  }
  std::vector<int32_t> split(static_cast<size_t>(cp) * cp);
  if (host_split &&
      hipMemcpyAsync(split.data(), route->dev.split, split.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return THD_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return THD_ERR_HIP;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t next_a = i + 1 < n ? a[i + 1].out : total;
    const int64_t next_b = i + 1 < n ? b[i + 1].out : total;
    if (host_runs_by_src) {  // out = zigzag row, in = token
      host_runs_by_src[3 * i + 0] = a[i].out;
      host_runs_by_src[3 * i + 1] = a[i].in;
      host_runs_by_src[3 * i + 2] = static_cast<int32_t>(next_a - a[i].out);
    }
    if (host_runs_by_dst) {  // out = token, in = zigzag row
      host_runs_by_dst[3 * i + 0] = b[i].in;
      host_runs_by_dst[3 * i + 1] = b[i].out;
      host_runs_by_dst[3 * i + 2] = static_cast<int32_t>(next_b - b[i].out);
    }
  }
  if (host_split) std::memcpy(host_split, split.data(), split.size() * 4);
  return THD_OK;
}

int thd_route_info(const thd_route* route, int32_t* cp_size, int64_t* total_tokens, int32_t* n_slots,
                   int32_t* built) {
  if (!route) return THD_ERR_ARG;
  if (cp_size) *cp_size = route->cp;
  if (total_tokens) *total_tokens = route->total;
  if (n_slots) *n_slots = route->n_slots;
  if (built) *built = route->built;
  return THD_OK;
}

int thd_route_launch_shape(thd_route* route, int64_t tile_bytes, int32_t nontemporal, int32_t block_threads,
                           int32_t tile_order) {
  if (!route || tile_bytes < 0 || nontemporal < 0 || nontemporal > 1 || tile_order < 0) return THD_ERR_ARG;
  if (block_threads != 0 && block_threads != 128 && block_threads != 256 && block_threads != 512 &&
      block_threads != 1024)
    return THD_ERR_ARG;
  route->launch = thdcp::SwapLaunch{tile_bytes, nontemporal, block_threads, tile_order};
  return THD_OK;
}

}  // extern "C"
