// Route construction on the GPU: zigzag <-> contiguous runs by interval
// intersection, with no host round trip.
//
// Method (Relax PR #273 "fla mcore chunkwise cp stage 3", §2.1): both layouts
// are unions of global token intervals -- one interval per rank for the
// contiguous layout, two per document per rank for the zigzag layout -- so the
// whole exchange is an intersection of intervals instead of per-token index
// tensors.  The pages do this with Python integers on the host after one
// device-to-host copy of the boundaries; here it runs on the device, so the
// host never waits: in one workgroup, or in every workgroup of one launch
// redundantly when the result fits in LDS, or, for routes of many documents,
// spread over many workgroups that place each segment's runs in closed form.
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
#include "thd_device.h"
#include "thd_internal.h"

namespace thdcp {
namespace {

constexpr int kBuildThreads = 1024;
constexpr int kBuildWaves = kBuildThreads / 64;

struct Segment {
  int32_t tok;   // first global token
  int32_t src;   // first emulated zigzag row
  int32_t len;   // tokens
  int32_t rank;  // zigzag (source) rank
};

// Compacted document k: start token a_k, chunk length c_k = L_k / (2 cp) and
// its local row in every rank's zigzag share, a_k / cp.  Stored as three
// arrays of `cap` entries: [start | chunk | offset].
struct Doc {
  int32_t a, c, off;
};

__device__ __forceinline__ Doc load_doc(const int32_t* docs, int32_t cap, int32_t k) {
  return Doc{docs[k], docs[cap + k], docs[2 * cap + k]};
}

// Chunk q of a document as a zigzag segment.
__device__ __forceinline__ Segment chunk_segment(const Doc& d, int32_t q, int32_t cp, int32_t share) {
  const bool back = q >= cp;
  Segment s;
  s.rank = back ? 2 * cp - 1 - q : q;
  s.tok = d.a + q * d.c;
  s.src = s.rank * share + d.off + (back ? d.c : 0);
  s.len = d.c;
  return s;
}

// Cuts of a segment at the contiguous ranks' borders (multiples of `share`):
// first destination rank and 1 or 2 pieces (a chunk is at most half a share).
struct Cut {
  int32_t first_d, rem, pieces;
};

__device__ __forceinline__ Cut cut_segment(const Segment& s, int32_t share, const FastDiv& div_share) {
  Cut c;
  c.first_d = div_share(s.tok);
  c.rem = s.tok - c.first_d * share;
  c.pieces = (c.rem + s.len > share) ? 2 : 1;
  return c;
}

// The LDS split matrix is kept in several copies while the segments are
// counted: lane l adds into copy l mod copies, because the lanes of a wave
// mostly hit the same few (source, destination) entries and atomics from many
// lanes to one LDS address serialise.  The copies are summed afterwards.
constexpr int kSplitEntries = 1024;  // cp * cp * copies stays within this
__host__ __device__ inline int split_copies(int32_t cp, int32_t n_slots) {
  if (2LL * cp * n_slots <= 1024) return 1;  // one pass over the segments: few atomics to spread
  const int64_t sq = static_cast<int64_t>(cp) * cp;
  if (sq >= kSplitEntries) return 1;
  const int c = static_cast<int>(kSplitEntries / sq);
  return c > 16 ? 16 : c;
}

// The build kernel keeps the compacted documents and the split matrix (in
// split_copies(cp, n_slots) copies) in LDS when they fit in kBuildLdsBytes;
// otherwise it uses the route's global scratch and global atomics (same
// steps, slower).
constexpr int kBuildLdsBytes = 150 * 1024;  // of the 160 KiB a workgroup may hold on MI355X

// Fused build: when the runs of both orders fit in LDS as well, every
// workgroup of one launch builds the whole route in its own LDS (the work is
// small at these sizes and identical in every workgroup), workgroup 0 writes
// it out, and each workgroup then writes its share of the directory from its
// LDS copy.  One launch instead of build + directory, and no workgroup ever
// waits for another.
constexpr int kFusedMaxSegments = 16384;
constexpr int kDirPerFusedGroup = 1024;  // directory rows per workgroup and direction, below the cap
// Cap on the fused build's workgroups.  Each one builds the whole route in its
// own LDS, so past a couple per CU more of them only repeat that build: a
// batch of 2^31 tokens would otherwise launch 131072 of them.  Above the cap
// every workgroup writes an equal, larger share of the directory.
constexpr int kFusedMaxGroups = 512;

// Largest i in [lo, hi) with runs[i].out <= row, given runs[lo].out <= row.
__device__ __forceinline__ int32_t last_run_at_or_before(const RunPair* runs, int32_t lo, int32_t hi, int32_t row) {
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (runs[mid].out <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// last_run_at_or_before over two run tables at once, row_a in a and row_b
// in b, so the two searches' LDS loads are in flight together (tables of
// equal length take the same steps).  Requires a[0].out <= row_a and
// b[0].out <= row_b when the table is not empty; an empty table gives 0.
__device__ __forceinline__ void last_runs_at_or_before(const RunPair* a, int32_t na, int32_t row_a, const RunPair* b,
                                                       int32_t nb, int32_t row_b, int32_t* ka, int32_t* kb) {
  int32_t lo_a = 0, hi_a = na, lo_b = 0, hi_b = nb;
  while (hi_a - lo_a > 1 || hi_b - lo_b > 1) {
    const bool go_a = hi_a - lo_a > 1, go_b = hi_b - lo_b > 1;
    const int32_t mid_a = (lo_a + hi_a) >> 1, mid_b = (lo_b + hi_b) >> 1;
    const int32_t out_a = go_a ? a[mid_a].out : 0;
    const int32_t out_b = go_b ? b[mid_b].out : 0;
    if (go_a) {
      if (out_a <= row_a) lo_a = mid_a;
      else hi_a = mid_a;
    }
    if (go_b) {
      if (out_b <= row_b) lo_b = mid_b;
      else hi_b = mid_b;
    }
  }
  *ka = lo_a;
  *kb = lo_b;
}

// Directory entry of output row `row` (a multiple of kDirBlock) from a run
// table of one order, given the run k that holds it.
__device__ __forceinline__ DirEntry dir_entry(const RunPair* runs, int32_t k, int32_t n_runs, int32_t row,
                                              int32_t total) {
  const RunPair r = runs[k];
  DirEntry e;
  e.in = r.in + (row - r.out);
  e.run_end = k + 1 < n_runs ? runs[k + 1].out : total;
  e.run = k;
  e.starts = 0;
  for (int32_t j = k + 1; j < n_runs && runs[j].out < row + kDirBlock; ++j) e.starts |= 1u << (runs[j].out - row);
  return e;
}

// Phases 1 and 2 of every build, in one pass over the boundaries: each
// boundary rule is checked (the severity of the worst rule a thread sees goes
// to *s_sev; precedence start, monotone, total, divisibility) and the
// non-empty slots go to `docs` as [start | chunk | local offset], `cap`
// entries per array, placed by a one-barrier scan per 1024 slots.  Every
// thread of the workgroup calls it; it returns the number of documents.  The
// caller publishes docs and *s_sev with a barrier.  on_doc(k, a, len) runs in
// the thread that places document k (also for boundaries that later fail
// validation: it must keep its own accesses in bounds).
template <typename OnDoc>
__device__ __forceinline__ int32_t compact_documents(const int32_t* __restrict__ cu, int32_t n_slots, int32_t cp,
                                                     int32_t total, int32_t* docs, int32_t cap, int32_t* s_wave1,
                                                     int* s_sev, OnDoc on_doc) {
  const int tid = threadIdx.x;
  int sev = 0;
  if (tid == 0) {
    if (cu[0] != 0) sev = kSevStart;
    if (cu[n_slots] != total) sev = max(sev, kSevTotal);
  }
  const int32_t two_cp = 2 * cp;
  int32_t n_docs = 0;
  for (int32_t base = 0; base < n_slots; base += kBuildThreads) {
    const int32_t i = base + tid;
    int32_t a = 0, len = 0;
    if (i < n_slots) {
      a = cu[i];
      const int64_t d = static_cast<int64_t>(cu[i + 1]) - a;
      if (d < 0) sev = max(sev, kSevMonotone);
      else if (d % two_cp != 0) sev = max(sev, kSevDivisible);
      else len = static_cast<int32_t>(d);
    }
    int32_t sum;
    const int32_t off =
        block_exclusive_scan_1b<kBuildThreads>(len > 0 ? 1 : 0, s_wave1, (base / kBuildThreads) & 1, &sum);
    if (len > 0) {
      const int32_t k = n_docs + off;
      docs[k] = a;
      docs[cap + k] = len / two_cp;
      docs[2 * cap + k] = a / cp;
      on_doc(k, a, len);
    }
    n_docs += sum;
  }
  if (sev) atomicMax(s_sev, sev);
  return n_docs;
}

// Header of a route whose boundaries failed validation (no runs).
__device__ __forceinline__ void write_failed_header(const RouteDev& ws, int32_t cp, int32_t total, int sev) {
  ws.hdr[kHdrRunsSrc] = 0;
  ws.hdr[kHdrRunsDst] = 0;
  ws.hdr[kHdrDocs] = 0;
  ws.hdr[kHdrCp] = cp;
  ws.hdr[kHdrTotal] = total;
  ws.hdr[kHdrStatus] = severity_to_code(sev);
}

template <bool kLds, bool kFused>
__global__ __launch_bounds__(kBuildThreads) void route_build_kernel(const int32_t* __restrict__ cu, int32_t n_slots,
                                                                    int32_t cp, int32_t total, RouteDev ws,
                                                                    int32_t lds_run_cap, FastDiv div_share,
                                                                    FastDiv div_two_cp, int32_t dir_per_group) {
  // kLds: docs[3 * n_slots], split[copies * cp * cp]; kFused adds, 8-byte
  // aligned, runs by zigzag row [lds_run_cap] and runs by token [lds_run_cap]
  extern __shared__ int32_t s_dyn[];
  __shared__ int32_t s_wave1[2 * kBuildWaves];  // the compaction passes' double-buffered scan
  __shared__ int32_t s_wave2[2 * kBuildWaves];  // the segment passes' double-buffered scan
  __shared__ int s_sev;
  const int tid = threadIdx.x;
  const bool writer = !kFused || blockIdx.x == 0;  // the workgroup that writes the route out
  const int32_t cap = kLds ? n_slots : ws.docs_cap;
  const int32_t cp2 = cp * cp;
  const int copies = kLds ? split_copies(cp, n_slots) : 1;
  int32_t* docs = kLds ? s_dyn : ws.docs;
  int32_t* split = kLds ? s_dyn + 3 * n_slots : ws.split;
  int32_t* my_split = split + (threadIdx.x & 63) % copies * cp2;  // this lane's copy
  RunPair* l_src = reinterpret_cast<RunPair*>(s_dyn + ((3 * n_slots + copies * cp2 + 1) & ~1));
  RunPair* l_dst = l_src + lds_run_cap;

  if (tid == 0) s_sev = 0;
  for (int i = tid; i < copies * cp2; i += kBuildThreads) {
    if constexpr (kLds) split[i] = 0;
    else __hip_atomic_store(&split[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- 1+2. validate and compact ----
  const int32_t two_cp = 2 * cp;
  const int32_t n_docs =
      compact_documents(cu, n_slots, cp, total, docs, cap, s_wave1, &s_sev, [](int32_t, int32_t, int32_t) {});
  if constexpr (!kLds) __threadfence();  // global path: zeroed split and document list are complete
  __syncthreads();                       // publishes the document list to the whole workgroup
  if (s_sev) {
    if (tid == 0 && writer) write_failed_header(ws, cp, total, s_sev);
    return;
  }

  // Valid boundaries: T is a multiple of 2*cp and every segment holds at least
  // one token, so the 2*cp*n_docs segment indices fit in int32.
  const int32_t share = total / cp;
  const int32_t n_seg = two_cp * n_docs;
  const int32_t two_n = 2 * n_docs;
  bool overflow = false;
  // segment j of the zigzag-row order is (rank r, position rem in the rank's
  // 2 * n_docs chunks); j grows by kBuildThreads per pass, so r and rem are
  // stepped instead of divided again (the other divisions, by share and by
  // 2 * cp, use the host's multiply-high constants)
  const int32_t step_r = n_seg > 0 ? kBuildThreads / two_n : 0;
  const int32_t step_rem = n_seg > 0 ? kBuildThreads - step_r * two_n : 0;
  int32_t r_j = n_seg > 0 ? tid / two_n : 0;
  int32_t rem_j = n_seg > 0 ? tid - r_j * two_n : 0;

  // ---- 3+4. runs in zigzag-row order (with the split matrix) and in token
  //           order.  Thread j looks at segment j of each order, counts the
  //           runs that start in it, and one scan of both counts (packed
  //           into 16-bit halves: at most 2048 per pass) places them. ----
  int32_t n_src = 0, n_dst = 0;
  for (int32_t base = 0; base < n_seg; base += kBuildThreads) {
    const int32_t j = base + tid;
    const int32_t r = r_j, rem = rem_j;  // j = r * two_n + rem
    if (base + kBuildThreads < n_seg) {
      r_j += step_r;
      rem_j += step_rem;
      if (rem_j >= two_n) {
        rem_j -= two_n;
        ++r_j;
      }
    }
    int32_t merge_s = 0, merge_t = 0;
    Segment ss{}, st{};
    Cut cs{0, 0, 0}, ct{0, 0, 0};
    if (j < n_seg) {
      // zigzag-row order: rank-major, then document, then front/back chunk
      const int32_t k = rem >> 1;
      const bool back = rem & 1;
      const Doc dk = load_doc(docs, cap, k);
      ss = chunk_segment(dk, back ? two_cp - 1 - r : r, cp, share);
      cs = cut_segment(ss, share, div_share);
      // Merges, in closed form.  The compacted documents lie end to end
      // (a_k = a_{k-1} + 2 cp c_{k-1}, every c > 0), so in rank r's share a
      // back chunk continues the tokens of the front chunk before it only
      // when r + 1 = 2 cp - 1 - r, i.e. r = cp - 1, and a front chunk those
      // of the previous document's back chunk (which ends at a_k - r c_{k-1})
      // only when r = 0.  A segment on a destination border starts a run.
      if (rem > 0 && cs.rem != 0) merge_s = (back ? r == cp - 1 : r == 0) ? 1 : 0;
      // token order: document-major, then chunk
      const int32_t kt = div_two_cp(j);
      const int32_t q = j - kt * two_cp;
      const Doc dt = load_doc(docs, cap, kt);
      st = chunk_segment(dt, q, cp, share);
      ct = cut_segment(st, share, div_share);
      // In token order chunk q continues the zigzag rows of the chunk before
      // it only where both sit in one rank's share back to back: chunk cp
      // after chunk cp - 1 (rank cp - 1, front then back of one document) and
      // chunk 0 after the previous document's chunk 2 cp - 1 (rank 0, whose
      // back chunk ends at row a_k / cp).  Any other neighbour lies in another
      // rank's share or, for two back chunks, c + share rows apart.
      if (ct.rem != 0) merge_t = (q == cp || (q == 0 && kt > 0)) ? 1 : 0;
    }
    const int count_s = j < n_seg ? cs.pieces - merge_s : 0;
    const int count_t = j < n_seg ? ct.pieces - merge_t : 0;
    int32_t sum;
    const int32_t off = block_exclusive_scan_1b<kBuildThreads>(count_s | (count_t << 16), s_wave2,
                                                               (base / kBuildThreads) & 1, &sum);
    if (j < n_seg) {
      const int32_t off_s = off & 0xFFFF, off_t = off >> 16;
      for (int p = 0; p < cs.pieces; ++p) {
        const int32_t ptok = p == 0 ? ss.tok : (cs.first_d + p) * share;
        const int32_t pend = min(ss.tok + ss.len, (cs.first_d + p + 1) * share);
        atomicAdd(&my_split[ss.rank * cp + cs.first_d + p], pend - ptok);
        if (p >= merge_s) {
          const int64_t slot = static_cast<int64_t>(n_src) + off_s + p - merge_s;
          const RunPair run{ss.src + (ptok - ss.tok), ptok};
          if (slot >= ws.run_cap || (kFused && slot >= lds_run_cap)) overflow = true;
          else {
            if (writer) ws.runs_src[slot] = run;
            if constexpr (kFused) l_src[slot] = run;
          }
        }
      }
      for (int p = merge_t; p < ct.pieces; ++p) {
        const int32_t ptok = p == 0 ? st.tok : (ct.first_d + p) * share;
        const int64_t slot = static_cast<int64_t>(n_dst) + off_t + p - merge_t;
        const RunPair run{ptok, st.src + (ptok - st.tok)};
        if (slot >= ws.run_cap || (kFused && slot >= lds_run_cap)) overflow = true;
        else {
          if (writer) ws.runs_dst[slot] = run;
          if constexpr (kFused) l_dst[slot] = run;
        }
      }
    }
    n_src += sum & 0xFFFF;
    n_dst += sum >> 16;
  }
  if constexpr (!kLds) __threadfence();  // global path: every split atomic has landed
  __syncthreads();
  if (copies > 1) {  // fold the copies into the first
    for (int i = tid; i < cp2; i += kBuildThreads) {
      int32_t v = split[i];
      for (int c = 1; c < copies; ++c) v += split[c * cp2 + i];
      split[i] = v;
    }
    __syncthreads();
  }

  if constexpr (kFused) {
    // ---- 5. this workgroup's share of the directory, both directions.  It
    //         is written before the integrity check: a route that fails the
    //         check gets an error status, and a failed route is never read
    //         past its status.  The counts are clamped to the LDS tables so
    //         no search leaves them even then. ----
    const int32_t nd = min(n_dst, lds_run_cap), ns = min(n_src, lds_run_cap);
    const int32_t n_blocks = (total + kDirBlock - 1) / kDirBlock;
    const int32_t b0 = static_cast<int32_t>(min(static_cast<int64_t>(blockIdx.x) * dir_per_group,
                                                static_cast<int64_t>(n_blocks)));
    const int32_t b1 = static_cast<int32_t>(min(static_cast<int64_t>(n_blocks), static_cast<int64_t>(b0) + dir_per_group));
    for (int32_t b = b0 + tid; b < b1; b += kBuildThreads) {
      const int32_t row = b << kDirShift;
      int32_t kd, ks;
      last_runs_at_or_before(l_dst, nd, row, l_src, ns, row, &kd, &ks);
      ws.dir_dst[b] = dir_entry(l_dst, kd, nd, row, total);
      ws.dir_src[b] = dir_entry(l_src, ks, ns, row, total);
    }
  }

  // ---- 6. integrity: same run count both ways; each rank sends and receives T/cp ----
  bool bad = overflow || n_src != n_dst;
  for (int i = tid; i < cp; i += kBuildThreads) {
    int64_t row = 0, col = 0;
    for (int d = 0; d < cp; ++d) {
      if constexpr (kLds) {
        row += split[i * cp + d];
        col += split[d * cp + i];
      } else {
        row += __hip_atomic_load(&split[i * cp + d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        col += __hip_atomic_load(&split[d * cp + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (row != share || col != share) bad = true;
  }
  if constexpr (kLds) {
    if (writer)
      for (int i = tid; i < cp * cp; i += kBuildThreads) ws.split[i] = split[i];
  }
  if (bad) atomicMax(&s_sev, 1);
  __syncthreads();
  if (tid == 0 && writer) {
    ws.hdr[kHdrRunsSrc] = n_src;
    ws.hdr[kHdrRunsDst] = n_dst;
    ws.hdr[kHdrDocs] = n_docs;
    ws.hdr[kHdrCp] = cp;
    ws.hdr[kHdrTotal] = total;
    ws.hdr[kHdrStatus] = s_sev ? THD_ERR_INTEGRITY : THD_OK;
  }
}

// Route build with run slots in closed form, for routes of more than one
// pass of segments (the threshold is on the host).  With the documents end
// to end, the runs that the segments before segment j of an order produce
// number j (one each), less the merges the rules above make among them, plus
// one for every destination border that falls strictly inside one of them
// (a second piece) or on the start of one the rules would have merged (a
// merge that does not happen).  The merges before j follow from j alone, and
// the cp - 1 borders are located once per workgroup, so every thread places
// the runs of its own segment of each order with no scan over the segments
// before it, and the segments spread over many workgroups.  One more workgroup, with no
// segments of its own, writes the split matrix, in closed form as well (per
// destination share, the chunks of the two documents at its ends plus 2 c
// for every document between them), checks it and writes the header.  The
// directory comes from the same launch or from route_index_kernel (below).
constexpr int kClosedMaxCp = 64;

// Rule merges among token-order segments before segment (document kt, chunk q):
// at chunk cp of every document and at chunk 0 of every document after the first.
__device__ __forceinline__ int32_t merges_before_token_order(int32_t kt, int32_t q, int32_t cp) {
  return (kt >= 1 ? 2 * kt - 1 : 0) + (kt >= 1 && q > 0 ? 1 : 0) + (q > cp ? 1 : 0);
}

// Rule merges among zigzag-row-order segments before segment (rank r,
// position rem): front chunks of documents 1.. on rank 0, back chunks on
// rank cp - 1.  r == cp stands for the end of the order.
__device__ __forceinline__ int32_t merges_before_zigzag_order(int32_t r, int32_t rem, int32_t cp, int32_t n_docs) {
  if (r >= cp) return 2 * n_docs - 1;
  if (r == 0) return rem >= 1 ? (rem - 1) >> 1 : 0;
  if (r < cp - 1) return n_docs - 1;
  return n_docs - 1 + (rem >> 1);
}

// Tokens of rank s's two chunks of document k inside [lo, hi).
__device__ __forceinline__ int32_t rank_tokens_in(const int32_t* docs, int32_t cap, int32_t k, int32_t s, int32_t cp,
                                                  int32_t lo, int32_t hi) {
  const int32_t a = docs[k], c = docs[cap + k];
  int32_t n = 0;
  for (int h = 0; h < 2; ++h) {
    const int32_t x0 = a + (h ? 2 * cp - 1 - s : s) * c;
    n += max(0, min(x0 + c, hi) - max(x0, lo));
  }
  return n;
}

// Runs that segment j of each order starts (n = 0, 1 or 2), at their global
// slots; two named fields rather than an array, so nothing is indexed at run
// time and the pair stays in registers.
struct SegmentRuns {
  RunPair run0, run1;
  int32_t slot0, slot1;
  int n;
};

// The runs a cut segment starts: its first piece unless it merges into the
// run before, and the piece after a destination border inside it.
__device__ __forceinline__ SegmentRuns segment_runs(int32_t base, int merge, int pieces, RunPair first,
                                                    RunPair second) {
  SegmentRuns out;
  out.n = 0;
  out.run0 = first;
  out.slot0 = base;
  out.run1 = second;
  out.slot1 = base + 1 - merge;
  if (!merge) out.n = 1;
  if (pieces == 2) {
    if (merge) {
      out.run0 = second;
      out.slot0 = out.slot1;
    }
    ++out.n;
  }
  return out;
}

// The border entries of one order whose key is below `key` (the key of a
// segment, in the form the table uses).  The table holds kClosedMaxCp
// entries (16-byte aligned), those of no border INT32_MAX, so the count runs
// over whole blocks of 8 entries: two 16-byte LDS reads in flight together
// instead of a dependent read per border.
__device__ __forceinline__ int32_t borders_before(const int32_t* s_border, int32_t cp, int32_t key) {
  const int32_t n_pad = (cp - 1 + 7) & ~7;
  int32_t n = 0;
  for (int32_t b0 = 0; b0 < n_pad; b0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) n += s_border[b0 + u] < key ? 1 : 0;
  }
  return n;
}

// Segment j of the zigzag-row order (rank r = j / (2 n_docs), then
// document, then front/back chunk) and the runs it starts; its border key is
// r * zz_stride + rem.
__device__ __forceinline__ SegmentRuns zigzag_segment_runs(const int32_t* docs, int32_t cap, int32_t n_docs, int32_t cp,
                                                           int32_t share, const FastDiv& div_share,
                                                           const int32_t* s_border, int32_t zz_stride, int32_t j) {
  const int32_t two_n = 2 * n_docs;
  const int32_t r = j / two_n, rem = j - r * two_n;
  const int32_t k = rem >> 1;
  const bool back = rem & 1;
  const Segment ss = chunk_segment(load_doc(docs, cap, k), back ? 2 * cp - 1 - r : r, cp, share);
  const Cut cs = cut_segment(ss, share, div_share);
  const int merge = (rem > 0 && cs.rem != 0 && (back ? r == cp - 1 : r == 0)) ? 1 : 0;
  const int32_t base =
      j - merges_before_zigzag_order(r, rem, cp, n_docs) + borders_before(s_border, cp, r * zz_stride + rem);
  const int32_t border = (cs.first_d + 1) * share;
  return segment_runs(base, merge, cs.pieces, RunPair{ss.src, ss.tok}, RunPair{ss.src + (border - ss.tok), border});
}

// Segment j of the token order (document j / (2 cp), then chunk) and the runs
// it starts.
__device__ __forceinline__ SegmentRuns token_segment_runs(const int32_t* docs, int32_t cap, int32_t cp, int32_t share,
                                                          const FastDiv& div_share, const FastDiv& div_two_cp,
                                                          const int32_t* s_border, int32_t j) {
  const int32_t two_cp = 2 * cp;
  const int32_t kt = div_two_cp(j), q = j - kt * two_cp;
  const Segment st = chunk_segment(load_doc(docs, cap, kt), q, cp, share);
  const Cut ct = cut_segment(st, share, div_share);
  const int merge = (ct.rem != 0 && (q == cp || (q == 0 && kt > 0))) ? 1 : 0;
  const int32_t base = j - merges_before_token_order(kt, q, cp) + borders_before(s_border, cp, j);
  const int32_t border = (ct.first_d + 1) * share;
  return segment_runs(base, merge, ct.pieces, RunPair{st.tok, st.src}, RunPair{border, st.src + (border - st.tok)});
}

// With kDir, each workgroup also writes the directory rows that start inside
// its own segments (a contiguous range of output rows in each order).  It
// keeps the runs of its segments in LDS, with those of the segment before
// (the run holding its first row may start there: runs never span more than
// two segments, as no two consecutive segments both merge) and of the
// kDirLookahead segments after (a 16-row block reaches at most 16 one-row
// segments further, and the run after the last one starts at most two
// segments on), so every search, run end and run-start bit comes from the
// table; entries carry global run indices.
constexpr int kDirLookahead = 18;
// Most own segments per workgroup, so that they, the one before and the
// lookahead fill one pass of the workgroup's threads.
constexpr int kMaxOwnSegments = kBuildThreads - 1 - kDirLookahead;
// Runs in each order's LDS table for `own` segments per workgroup: at most
// two per segment.
__host__ __device__ inline int32_t dir_table_runs(int32_t own) { return 2 * (own + 1 + kDirLookahead); }

// `own`: segments per workgroup (at most kMaxOwnSegments with kDir, at most
// kBuildThreads without).
template <bool kDir>
__global__ __launch_bounds__(kBuildThreads) void route_runs_kernel(const int32_t* __restrict__ cu, int32_t n_slots,
                                                                   int32_t cp, int32_t total, RouteDev ws,
                                                                   FastDiv div_share, FastDiv div_two_cp,
                                                                   int32_t own) {
  // docs [3 * n_slots], split [cp * cp] (the writer), then, 8-byte aligned
  // and with kDir, the runs of each order [dir_table_runs(own)] each
  extern __shared__ int32_t s_dyn[];
  __shared__ int32_t s_wave1[2 * kBuildWaves];
  __shared__ int s_sev;
  // Border b + 1's key in each order where it adds a run, else INT32_MAX:
  // token order, its segment's index; zigzag-row order, r * zz_stride + rem
  // for its segment (rank r, position rem), with zz_stride = 2 * n_slots >=
  // 2 * n_docs, so keys sort as the segment indices do while the number of
  // documents is not yet known.
  __shared__ __align__(16) int32_t s_border_s[kClosedMaxCp];
  __shared__ __align__(16) int32_t s_border_t[kClosedMaxCp];
  __shared__ int32_t s_end_doc[kClosedMaxCp];  // document holding token d * share (the writer)
  const int tid = threadIdx.x;
  // the last workgroup has no segments of its own: it writes the split
  // matrix and the header while the others place runs
  const bool writer = blockIdx.x == gridDim.x - 1;
  const int32_t cap = n_slots;
  int32_t* docs = s_dyn;
  RunPair* l_src = reinterpret_cast<RunPair*>(s_dyn + ((3 * n_slots + cp * cp + 1) & ~1));
  const int32_t table_runs = dir_table_runs(own);
  RunPair* l_dst = l_src + table_runs;
  const int32_t share = total / cp, two_cp = 2 * cp, zz_stride = 2 * n_slots;
  if (tid == 0) s_sev = 0;
  if (tid < kClosedMaxCp) {
    s_border_s[tid] = INT32_MAX;
    s_border_t[tid] = INT32_MAX;
  }

  // ---- 1+2+3. validate and compact (every workgroup), and the destination
  //             borders b * share, b = 0 .. cp-1, from the document each
  //             falls in: the documents lie end to end from token 0 to T, so
  //             the thread placing document k takes the borders inside
  //             [a_k, a_k + 2 cp c_k) and records, per order, the key of
  //             each (b >= 1) where it adds a run; the writer also keeps the
  //             document of every border.  A document outside [0, T) (only
  //             on boundaries that fail validation) records nothing. ----
  auto place_borders = [&](int32_t k, int32_t a, int32_t len) {
    if (a < 0 || static_cast<int64_t>(a) + len > total) return;
    const int32_t c = len / two_cp, end = a + len;
    int32_t b = div_share(a);
    if (b * share < a) ++b;
    for (; b < cp && b * share < end; ++b) {
      if (writer) s_end_doc[b] = k;
      if (b == 0) continue;
      const int32_t t = b * share;
      const int32_t q = (t - a) / c;
      const bool inside = t - a != q * c;
      const bool back = q >= cp;
      const int32_t r = back ? two_cp - 1 - q : q, rem = 2 * k + (back ? 1 : 0);
      const bool rule_s = rem > 0 && (back ? r == cp - 1 : r == 0);
      const bool rule_t = q == cp || (q == 0 && k > 0);
      s_border_s[b - 1] = (inside || rule_s) ? r * zz_stride + rem : INT32_MAX;
      s_border_t[b - 1] = (inside || rule_t) ? k * two_cp + q : INT32_MAX;
    }
  };
  const int32_t n_docs = compact_documents(cu, n_slots, cp, total, docs, cap, s_wave1, &s_sev, place_borders);
  __syncthreads();
  if (s_sev) {
    if (tid == 0 && writer) write_failed_header(ws, cp, total, s_sev);
    return;
  }
  // valid boundaries and total > 0 (the host's launch condition): n_docs >= 1
  const int32_t two_n = 2 * n_docs, n_seg = two_cp * n_docs;

  // ---- 4. this workgroup's segments of each order (with kDir, and the
  //         neighbours its directory rows need, into LDS) ----
  const int32_t j_lo = static_cast<int32_t>(min(static_cast<int64_t>(blockIdx.x) * own, static_cast<int64_t>(n_seg)));
  const int32_t j_hi = min(n_seg, j_lo + own);
  const int32_t t_lo = kDir ? max(0, j_lo - 1) : j_lo;
  const int32_t t_hi = kDir ? min(n_seg, j_hi + kDirLookahead) : j_hi;
  // global slot of the table's first run, per order
  int32_t base_s = 0, base_t = 0;
  if constexpr (kDir) {
    if (t_lo < n_seg) {
      const int32_t r = t_lo / two_n, rem = t_lo - r * two_n;
      base_s = t_lo - merges_before_zigzag_order(r, rem, cp, n_docs) +
               borders_before(s_border_s, cp, r * zz_stride + rem);
      const int32_t kt = div_two_cp(t_lo), q = t_lo - kt * two_cp;
      base_t = t_lo - merges_before_token_order(kt, q, cp) + borders_before(s_border_t, cp, t_lo);
    }
  }
  for (int32_t j = t_lo + tid; j < t_hi; j += kBuildThreads) {
    const bool own = j >= j_lo && j < j_hi;
    const SegmentRuns zs = zigzag_segment_runs(docs, cap, n_docs, cp, share, div_share, s_border_s, zz_stride, j);
    const SegmentRuns ts = token_segment_runs(docs, cap, cp, share, div_share, div_two_cp, s_border_t, j);
    if (own) {
      if (zs.n > 0 && zs.slot0 < ws.run_cap) ws.runs_src[zs.slot0] = zs.run0;
      if (zs.n > 1 && zs.slot1 < ws.run_cap) ws.runs_src[zs.slot1] = zs.run1;
      if (ts.n > 0 && ts.slot0 < ws.run_cap) ws.runs_dst[ts.slot0] = ts.run0;
      if (ts.n > 1 && ts.slot1 < ws.run_cap) ws.runs_dst[ts.slot1] = ts.run1;
    }
    if constexpr (kDir) {
      const int32_t ls0 = zs.slot0 - base_s, ls1 = zs.slot1 - base_s;
      const int32_t lt0 = ts.slot0 - base_t, lt1 = ts.slot1 - base_t;
      if (zs.n > 0 && ls0 >= 0 && ls0 < table_runs) l_src[ls0] = zs.run0;
      if (zs.n > 1 && ls1 >= 0 && ls1 < table_runs) l_src[ls1] = zs.run1;
      if (ts.n > 0 && lt0 >= 0 && lt0 < table_runs) l_dst[lt0] = ts.run0;
      if (ts.n > 1 && lt1 >= 0 && lt1 < table_runs) l_dst[lt1] = ts.run1;
    }
  }
  if constexpr (kDir) {
    // runs in the tables: the runs before t_hi less those before t_lo
    int32_t end_s = 0, end_t = 0;
    if (t_hi < n_seg) {
      const int32_t r = t_hi / two_n, rem = t_hi - r * two_n;
      end_s = t_hi - merges_before_zigzag_order(r, rem, cp, n_docs) +
              borders_before(s_border_s, cp, r * zz_stride + rem);
      const int32_t kt = div_two_cp(t_hi), q = t_hi - kt * two_cp;
      end_t = t_hi - merges_before_token_order(kt, q, cp) + borders_before(s_border_t, cp, t_hi);
    } else {
      end_s = n_seg - merges_before_zigzag_order(cp, 0, cp, n_docs) + borders_before(s_border_s, cp, INT32_MAX);
      end_t = n_seg - merges_before_token_order(n_docs, 0, cp) + borders_before(s_border_t, cp, INT32_MAX);
    }
    const int32_t n_ls = min(end_s - base_s, table_runs), n_lt = min(end_t - base_t, table_runs);
    __syncthreads();
    // ---- 5. the directory rows that start inside this workgroup's segments ----
    if (j_lo < n_seg) {
      // first output row of segment j in each order (total past the last)
      auto first_row_s = [&](int32_t j) -> int32_t {
        if (j >= n_seg) return total;
        const int32_t r = j / two_n, rem = j - r * two_n;
        const Doc d = load_doc(docs, cap, rem >> 1);
        return r * share + d.off + ((rem & 1) ? d.c : 0);
      };
      auto first_row_t = [&](int32_t j) -> int32_t {
        if (j >= n_seg) return total;
        const int32_t kt = div_two_cp(j), q = j - kt * two_cp;
        const Doc d = load_doc(docs, cap, kt);
        return d.a + q * d.c;
      };
      const int32_t s0 = (first_row_s(j_lo) + kDirBlock - 1) >> kDirShift, s1 = (first_row_s(j_hi) + kDirBlock - 1) >> kDirShift;
      const int32_t d0 = (first_row_t(j_lo) + kDirBlock - 1) >> kDirShift, d1 = (first_row_t(j_hi) + kDirBlock - 1) >> kDirShift;
      // entry i of each order in one step, both searches' LDS reads in
      // flight together (an order with no entry i searches an empty table)
      for (int32_t i = tid; i < max(s1 - s0, d1 - d0); i += kBuildThreads) {
        const bool has_s = s0 + i < s1, has_t = d0 + i < d1;
        const int32_t row_s = (s0 + i) << kDirShift, row_t = (d0 + i) << kDirShift;
        int32_t ks, kt;
        last_runs_at_or_before(l_src, has_s ? n_ls : 0, row_s, l_dst, has_t ? n_lt : 0, row_t, &ks, &kt);
        if (has_s) {
          DirEntry e = dir_entry(l_src, ks, n_ls, row_s, total);
          e.run += base_s;
          ws.dir_src[s0 + i] = e;
        }
        if (has_t) {
          DirEntry e = dir_entry(l_dst, kt, n_lt, row_t, total);
          e.run += base_t;
          ws.dir_dst[d0 + i] = e;
        }
      }
    }
  }
  if (!writer) return;

  // ---- 6. the writer workgroup: totals, split matrix, integrity, header ----
  int32_t* split = s_dyn + 3 * n_slots;
  for (int32_t e = tid; e < cp * cp; e += kBuildThreads) {
    const int32_t src = e / cp, d = e - src * cp;
    const int32_t lo = d * share, hi = lo + share;
    const int32_t k0 = s_end_doc[d];
    // the document holding token hi - 1: the one holding hi, or the one
    // before it when hi starts a document (hi > 0 = a_0, so that one exists)
    int32_t k1 = n_docs - 1;
    if (d + 1 < cp) {
      const int32_t k_hi = s_end_doc[d + 1];
      k1 = docs[k_hi] == hi ? k_hi - 1 : k_hi;
    }
    int32_t v = rank_tokens_in(docs, cap, k0, src, cp, lo, hi);
    // documents strictly between hold 2 c tokens of every rank; sum of c over
    // documents before k is a_k / (2 cp)
    if (k1 > k0) v += rank_tokens_in(docs, cap, k1, src, cp, lo, hi) + 2 * ((docs[k1] - docs[k0 + 1]) / two_cp);
    split[e] = v;
    ws.split[e] = v;
  }
  __syncthreads();
  int32_t extra_s = 0, extra_t = 0;
  for (int b = 0; b < cp - 1; ++b) {
    extra_s += s_border_s[b] != INT32_MAX ? 1 : 0;
    extra_t += s_border_t[b] != INT32_MAX ? 1 : 0;
  }
  const int64_t n_src = static_cast<int64_t>(n_seg) - merges_before_zigzag_order(cp, 0, cp, n_docs) + extra_s;
  const int64_t n_dst = static_cast<int64_t>(n_seg) - merges_before_token_order(n_docs, 0, cp) + extra_t;
  bool bad = n_src != n_dst || n_src > ws.run_cap;
  for (int i = tid; i < cp; i += kBuildThreads) {
    int64_t row = 0, col = 0;
    for (int d = 0; d < cp; ++d) {
      row += split[i * cp + d];
      col += split[d * cp + i];
    }
    if (row != share || col != share) bad = true;
  }
  if (bad) atomicMax(&s_sev, 1);
  __syncthreads();
  if (tid == 0) {
    ws.hdr[kHdrRunsSrc] = static_cast<int32_t>(min(n_src, ws.run_cap));
    ws.hdr[kHdrRunsDst] = static_cast<int32_t>(min(n_dst, ws.run_cap));
    ws.hdr[kHdrDocs] = n_docs;
    ws.hdr[kHdrCp] = cp;
    ws.hdr[kHdrTotal] = total;
    ws.hdr[kHdrStatus] = s_sev ? THD_ERR_INTEGRITY : THD_OK;
  }
}

// The same search done by one wave: each round, 64 lanes probe 64 evenly
// spaced runs and a ballot keeps the interval that holds the answer, so a
// list of up to 4096 runs takes two dependent loads instead of twelve.
__device__ __forceinline__ int32_t wave_last_run_at_or_before(const RunPair* runs, int32_t n, int32_t row,
                                                              int lane) {
  int32_t lo = 0, hi = n;  // runs[lo].out <= row (runs[0].out == 0); answer in [lo, hi)
  while (hi - lo > 1) {
    const int32_t step = (hi - lo + 63) / 64;
    const int32_t idx = lo + lane * step;
    const bool le = idx < hi && runs[idx].out <= row;
    const uint64_t m = __ballot(le);  // a prefix of the lanes; lane 0 is always set
    const int last = 63 - __clzll(static_cast<long long>(m));
    lo += last * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

constexpr int kIndexThreads = 256;   // four waves: one search each (2 directions x window ends)
constexpr int kIndexStage = 1024;    // runs of one window staged in LDS up to this many

// Directory: for every 16th output row of each direction, the input row that
// feeds it, the end of its run and the run index.  A workgroup covers 256
// directory rows; its four waves first find the runs at both ends of that row
// window (per direction), the window's runs are staged in LDS, and each
// thread then searches only that short list.
__global__ __launch_bounds__(kIndexThreads) void route_index_kernel(RouteDev ws, int32_t n_blocks, int32_t total) {
  __shared__ int32_t s_k[2][2];
  __shared__ RunPair s_runs[2][kIndexStage];
  if (ws.hdr[kHdrStatus] != THD_OK) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t b0 = blockIdx.x * kIndexThreads;
  const int32_t b_last = min(n_blocks, b0 + kIndexThreads) - 1;
  const int32_t n_runs[2] = {ws.hdr[kHdrRunsDst], ws.hdr[kHdrRunsSrc]};
  const RunPair* runs[2] = {ws.runs_dst, ws.runs_src};
  DirEntry* dir[2] = {ws.dir_dst, ws.dir_src};
  {
    const int d = wave >> 1;
    const int32_t row = (wave & 1) ? (b_last << kDirShift) : (b0 << kDirShift);
    const int32_t k = wave_last_run_at_or_before(runs[d], n_runs[d], row, lane);
    if (lane == 0) s_k[d][wave & 1] = k;
  }
  __syncthreads();
  bool staged[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int32_t k_lo = s_k[d][0];
    // the window's runs plus the kDirBlock after it: every run that starts
    // inside the window's last directory block, and the one after that
    const int32_t cnt = min(s_k[d][1] + kDirBlock + 1, n_runs[d]) - k_lo;
    staged[d] = cnt <= kIndexStage;
    if (staged[d])
      for (int i = tid; i < cnt; i += kIndexThreads) s_runs[d][i] = runs[d][k_lo + i];
  }
  __syncthreads();
  const int32_t b = b0 + tid;
  if (b >= n_blocks) return;
  const int32_t row = b << kDirShift;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int32_t k_lo = s_k[d][0], k_hi = s_k[d][1];
    DirEntry e;
    if (staged[d]) {
      const int32_t n_staged = min(k_hi + kDirBlock + 1, n_runs[d]) - k_lo;
      const int32_t k = last_run_at_or_before(s_runs[d], 0, k_hi - k_lo + 1, row);
      e = dir_entry(s_runs[d], k, n_staged, row, total);
      e.run += k_lo;
    } else {
      e = dir_entry(runs[d], last_run_at_or_before(runs[d], k_lo, k_hi + 1, row), n_runs[d], row, total);
    }
    dir[d][b] = e;
  }
}

}  // namespace

// Dynamic LDS of the build kernel: documents and split copies (int32), and,
// fused, the runs of both orders (8-byte aligned).
int64_t build_lds_bytes(int32_t n_slots, int32_t cp, bool fused) {
  const int64_t words = 3LL * n_slots + static_cast<int64_t>(split_copies(cp, n_slots)) * cp * cp;
  if (!fused) return 4 * words;
  return 4 * ((words + 1) & ~1LL) + 16 * (2LL * cp * n_slots + cp);
}

namespace {

// Routes of more than one pass of segments, cp <= kClosedMaxCp and
// documents plus split matrix in LDS: route_runs_kernel.  Measured on
// MI355X (same box, interleaved): 7.6 us for 1984 and for 3680 segments
// against 10.2 and 12.7 us for two and four passes of the one-pass build,
// 7.9 us for 8320 segments against 19.4 us for nine.
constexpr int64_t kClosedMinSegments = kBuildThreads;
constexpr int64_t kDirBlocksPerGroup = 2048;  // directory entries (16 rows each) per workgroup, on average, for the one-launch form
// Own segments per workgroup of the one-launch form: at least kMinOwnSegments,
// more once that many would take more than kClosedGroups workgroups (every
// workgroup validates and compacts the whole boundary list first).  A
// workgroup's segment and directory work is a chain of dependent LDS reads
// per thread, so fewer segments per workgroup over more CUs shorten it:
// 128 segments ran 8320 segments in 9.5 us against 11.5 us with 1005
// (64: the same, 256: 9.9 us).
constexpr int64_t kMinOwnSegments = 128;
constexpr int64_t kClosedGroups = 255;

// Only for total > 0: valid boundaries then hold at least one document,
// which the closed form's border and split steps need (an empty batch takes
// the one-pass build, where it is no work at all).
bool route_build_closed(int32_t n_slots, int32_t cp, int32_t total) {
  const int64_t segments = 2LL * cp * n_slots;
  return total > 0 && segments > kClosedMinSegments && cp <= kClosedMaxCp &&
         4 * (3LL * n_slots + static_cast<int64_t>(cp) * cp) <= kBuildLdsBytes;
}

bool route_build_fused(int32_t n_slots, int32_t cp) {
  const int64_t segments = 2LL * cp * n_slots;
  return segments <= kFusedMaxSegments && build_lds_bytes(n_slots, cp, true) <= kBuildLdsBytes;
}

}  // namespace

hipError_t launch_route_build(const int32_t* cu, int32_t n_slots, int32_t cp, int32_t total, const RouteDev& ws,
                              hipStream_t stream) {
  const int64_t lds = build_lds_bytes(n_slots, cp, false);
  const FastDiv div_share = FastDiv::make(total / cp > 0 ? total / cp : 1);
  const FastDiv div_two_cp = FastDiv::make(2 * cp);
  if (route_build_closed(n_slots, cp, total)) {
    const int64_t segments = 2LL * cp * n_slots;
    const int64_t grid = (segments + kBuildThreads - 1) / kBuildThreads;
    int64_t own = (segments + kClosedGroups - 1) / kClosedGroups;
    own = own < kMinOwnSegments ? kMinOwnSegments : (own > kMaxOwnSegments ? kMaxOwnSegments : own);
    const int64_t grid_dir = (segments + own - 1) / own;
    const int64_t words = 3LL * n_slots + static_cast<int64_t>(cp) * cp;
    const int64_t lds_runs = 4 * words;
    const int64_t lds_dir = 4 * ((words + 1) & ~1LL) +
                            2LL * dir_table_runs(static_cast<int32_t>(own)) * static_cast<int64_t>(sizeof(RunPair));
    const int64_t n_blocks = (static_cast<int64_t>(total) + kDirBlock - 1) / kDirBlock;
    // The directory in the same launch while the entries each workgroup's
    // segments cover stay few; past that the directory launch spreads them
    // over the whole chip.  One more workgroup than the segments fill: the
    // writer of the split matrix and header.
    if (n_blocks <= kDirBlocksPerGroup * grid_dir && lds_dir <= kBuildLdsBytes) {
      hipLaunchKernelGGL((route_runs_kernel<true>), dim3(static_cast<unsigned>(grid_dir + 1)), dim3(kBuildThreads),
                         static_cast<size_t>(lds_dir), stream, cu, n_slots, cp, total, ws, div_share, div_two_cp,
                         static_cast<int32_t>(own));
      return hipGetLastError();
    }
    hipLaunchKernelGGL((route_runs_kernel<false>), dim3(static_cast<unsigned>(grid + 1)), dim3(kBuildThreads),
                       static_cast<size_t>(lds_runs), stream, cu, n_slots, cp, total, ws, div_share, div_two_cp,
                       kBuildThreads);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_route_index(ws, total, stream);
  }
  if (route_build_fused(n_slots, cp)) {
    const int32_t run_cap = 2 * cp * n_slots + cp;
    const int64_t lds_fused = build_lds_bytes(n_slots, cp, true);
    const int32_t n_blocks = (total + kDirBlock - 1) / kDirBlock;
    int32_t grid = n_blocks > 0 ? (n_blocks + kDirPerFusedGroup - 1) / kDirPerFusedGroup : 1;
    if (grid > kFusedMaxGroups) grid = kFusedMaxGroups;
    const int32_t dir_per_group = n_blocks > 0 ? (n_blocks + grid - 1) / grid : kDirPerFusedGroup;
    hipLaunchKernelGGL((route_build_kernel<true, true>), dim3(grid), dim3(kBuildThreads),
                       static_cast<size_t>(lds_fused), stream, cu, n_slots, cp, total, ws, run_cap, div_share,
                       div_two_cp, dir_per_group);
    return hipGetLastError();
  }
  if (lds <= kBuildLdsBytes)
    hipLaunchKernelGGL((route_build_kernel<true, false>), dim3(1), dim3(kBuildThreads), static_cast<size_t>(lds),
                       stream, cu, n_slots, cp, total, ws, 0, div_share, div_two_cp, 0);
  else
    hipLaunchKernelGGL((route_build_kernel<false, false>), dim3(1), dim3(kBuildThreads), 0, stream, cu, n_slots, cp,
                       total, ws, 0, div_share, div_two_cp, 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_route_index(ws, total, stream);
}

hipError_t launch_route_index(const RouteDev& ws, int32_t total, hipStream_t stream) {
  const int32_t n_blocks = (total + kDirBlock - 1) / kDirBlock;
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(route_index_kernel, dim3((n_blocks + kIndexThreads - 1) / kIndexThreads), dim3(kIndexThreads), 0,
                     stream, ws, n_blocks, total);
  return hipGetLastError();
}

}  // namespace thdcp
