// Document-aware label shift, MTP roll and valid-token mask in one pass.
//
// Page "Packed Sequence 与上下文并行": labels are the next token, but never
// across a document (§1.3); each MTP depth needs the same care, one more
// token ahead (§1.6); pads added per document for alignment (§2.2) carry no
// label and are zero in the valid-token mask (§2.2, §3.4).  The pages do these
// with a Python loop over documents and a separate MTP helper; here one kernel
// writes every shifted stream and every mask.
//
// For position t in padded slot s, e = cu_pad[s] + real length of s is the end
// of the document's real tokens:
//   mask[0][t] = t < e
//   shifted[j-1][t] = ids[t+j] and mask[j][t] = 1 when t + j < e, else fill / 0.
//
// Each workgroup first checks the whole boundary lists (cheap: a few hundred
// ints from L2), so that a bad list stops every workgroup before it writes
// anything; it stages the boundaries in LDS when they fit and its slice of
// ids (plus max_shift tokens of look-ahead) in LDS, then gives each thread one
// position: a binary search finds the slot, and the J shifted values and J+1
// mask bytes are written with consecutive lanes on consecutive positions.
// The ids, and with a route its header and the directory entry of the
// thread's position, do not depend on the boundaries: they are read in the
// same memory round trip as the boundaries, before the checks.
#include "thd_internal.h"

namespace thdcp {
namespace {

constexpr int kRollThreads = 256;
constexpr int kRollLdsSlots = 4096;  // boundaries staged in LDS (dynamic, 8 B per slot, <= 32 KiB)

// Zigzag row of token t from a route's token-order runs (out = token, in =
// zigzag row), given e, the directory entry of t's 16-row block; every access
// stays in the run table.
__device__ __forceinline__ int32_t zigzag_row_of(const RollRoute& rt, const DirEntry& e, int32_t n_runs, int32_t t) {
  if (t < e.run_end) return e.in + (t & (kDirBlock - 1));
  const int32_t k = min(run_of_row(e, t), n_runs - 1);
  const RunPair r = rt.runs[k];
  return r.in + (t - r.out);
}

template <bool kLds, bool kRouted>
__global__ __launch_bounds__(kRollThreads) void roll_kernel(const int64_t* __restrict__ ids,
                                                            const int32_t* __restrict__ cu_pad,
                                                            const int32_t* __restrict__ cu_real, int32_t n_slots,
                                                            int32_t total, int32_t max_shift, int64_t fill,
                                                            int64_t* __restrict__ shifted,
                                                            uint8_t* __restrict__ mask, int32_t* __restrict__ status,
                                                            RollRoute rt) {
  extern __shared__ int32_t s_cu[];                   // kLds: [n_slots + 1] padded, then [n_slots] real lengths
  int32_t* s_pad = s_cu;
  int32_t* s_len = s_cu + (n_slots + 1);
  __shared__ int64_t s_ids[kRollThreads + THD_MAX_SHIFT];
  __shared__ int s_sev;
  const int tid = threadIdx.x;

  // reads that do not depend on the boundaries, issued with them
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRollThreads;
  const int n_load = t0 < total ? static_cast<int>(min(static_cast<int64_t>(total) - t0,
                                                        static_cast<int64_t>(kRollThreads + max_shift)))
                                : 0;
  int64_t id_own = 0, id_ahead = 0;  // ids[t0 + tid] and ids[t0 + kRollThreads + tid]
  if (tid < n_load) id_own = ids[t0 + tid];
  if (kRollThreads + tid < n_load) id_ahead = ids[t0 + kRollThreads + tid];
  const int64_t t = t0 + tid;
  int32_t route_status = THD_OK, n_runs = 0;
  DirEntry e_dir{};
  if constexpr (kRouted) {
    route_status = rt.hdr[kHdrStatus];
    n_runs = rt.hdr[kHdrRunsDst];
    if (t < total) e_dir = rt.dir[t >> kDirShift];
  }

  if (tid == 0) s_sev = 0;
  __syncthreads();
  int sev = 0;
  if (tid == 0) {
    if (cu_pad[0] != 0 || (cu_real && cu_real[0] != 0)) sev = kSevStart;
    if (cu_pad[n_slots] != total) sev = max(sev, kSevTotal);
  }
  for (int i = tid; i <= n_slots; i += kRollThreads) {
    const int32_t p0 = cu_pad[i];
    if constexpr (kLds) s_pad[i] = p0;
    if (i < n_slots) {
      const int32_t p1 = cu_pad[i + 1];
      const int64_t plen = static_cast<int64_t>(p1) - p0;
      int64_t rlen = plen;
      if (cu_real) rlen = static_cast<int64_t>(cu_real[i + 1]) - cu_real[i];
      if (plen < 0 || rlen < 0) sev = max(sev, kSevMonotone);
      else if (rlen > plen) sev = max(sev, kSevRealGtPadded);
      if constexpr (kLds) s_len[i] = static_cast<int32_t>(rlen);
    }
  }
  if (sev) atomicMax(&s_sev, sev);
  __syncthreads();
  int32_t code = severity_to_code(s_sev);
  if (kRouted && route_status != THD_OK) code = route_status;  // a failed route build comes first
  if (status && blockIdx.x == 0 && tid == 0) *status = code;
  if (code != THD_OK) return;

  if (t0 >= total) return;
  if (tid < n_load) s_ids[tid] = id_own;
  if (kRollThreads + tid < n_load) s_ids[kRollThreads + tid] = id_ahead;
  __syncthreads();

  if (t >= total) return;
  // slot s: cu_pad[s] <= t < cu_pad[s + 1]; that slot is never empty
  int32_t lo = 0, hi = n_slots;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    const int32_t v = kLds ? s_pad[mid] : cu_pad[mid];
    if (v <= t) lo = mid;
    else hi = mid;
  }
  int64_t real_len;
  if constexpr (kLds) real_len = s_len[lo];
  else real_len = cu_real ? static_cast<int64_t>(cu_real[lo + 1]) - cu_real[lo]
                          : static_cast<int64_t>(cu_pad[lo + 1]) - cu_pad[lo];
  const int64_t e = static_cast<int64_t>(kLds ? s_pad[lo] : cu_pad[lo]) + real_len;
  const int64_t row = kRouted ? zigzag_row_of(rt, e_dir, n_runs, static_cast<int32_t>(t)) : t;
  mask[row] = t < e ? 1 : 0;
  for (int j = 1; j <= max_shift; ++j) {
    const bool ok = t + j < e;
    shifted[static_cast<int64_t>(j - 1) * total + row] = ok ? s_ids[tid + j] : fill;
    mask[static_cast<int64_t>(j) * total + row] = ok ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_roll(const int64_t* ids, const int32_t* cu_pad, const int32_t* cu_real, int32_t n_slots,
                       int32_t total, int32_t max_shift, int64_t fill, int64_t* shifted, uint8_t* mask,
                       int32_t* status, const RollRoute* route, hipStream_t stream) {
  const int64_t blocks64 = total > 0 ? (static_cast<int64_t>(total) + kRollThreads - 1) / kRollThreads : 1;
  const dim3 grid(static_cast<unsigned>(blocks64));
  const RollRoute rt = route ? *route : RollRoute{nullptr, nullptr, nullptr};
  const bool lds = n_slots + 1 <= kRollLdsSlots;
  const size_t lds_bytes = lds ? static_cast<size_t>(2 * n_slots + 1) * 4 : 0;
#define THD_ROLL(L, R)                                                                                             \
  hipLaunchKernelGGL((roll_kernel<L, R>), grid, dim3(kRollThreads), lds_bytes, stream, ids, cu_pad, cu_real,      \
                     n_slots, total, max_shift, fill, shifted, mask, status, rt)
  if (lds) {
    if (route) THD_ROLL(true, true);
    else THD_ROLL(true, false);
  } else {
    if (route) THD_ROLL(false, true);
    else THD_ROLL(false, false);
  }
#undef THD_ROLL
  return hipGetLastError();
}

}  // namespace thdcp
