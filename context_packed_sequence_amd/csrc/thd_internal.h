// Internal declarations shared by the translation units of libthdcp.
// Not part of the public ABI (that is include/thd_cp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "thd_cp.h"

namespace thdcp {

// The run directory holds one entry per block of 1 << kDirShift rows.
constexpr int kDirShift = 4;
constexpr int kDirBlock = 1 << kDirShift;

// Header words of the route workspace (int32).
enum HeaderWord : int {
  kHdrStatus = 0,     // THD_OK or a THD_ERR_* code written by the build kernel
  kHdrRunsSrc = 1,    // runs in zigzag-row order
  kHdrRunsDst = 2,    // runs in token (contiguous-row) order
  kHdrDocs = 3,       // non-empty slots
  kHdrCp = 4,
  kHdrTotal = 5,
  kHdrWords = 16,
};

// A run maps `len` consecutive input rows onto `len` consecutive output rows.
// Stored as (first output row, first input row); the length is implied by the
// next run's output row (or the total for the last run), because the runs of
// one order tile the output rows without gaps.
struct RunPair {
  int32_t out;
  int32_t in;
};

// Directory entry for output row 16*b: everything a swap tile starting there
// needs to begin copying, in one 16-byte load.
struct DirEntry {
  int32_t in;       // input row that feeds output row 16*b
  int32_t run_end;  // first output row after the run that holds 16*b
  int32_t run;      // index of that run
  uint32_t starts;  // bit i (1..15): a run starts at output row 16*b + i
};

// Index of the run that holds output row r, from r's directory entry: the
// entry's run plus the runs that start inside the block at or before r.
__host__ __device__ inline int32_t run_of_row(const DirEntry& e, int32_t r) {
  const uint32_t upto = (2u << (r & (kDirBlock - 1))) - 1u;  // bits 0..(r mod 16)
  return e.run + __builtin_popcount(e.starts & upto & ~1u);
}

// Device pointers into the route workspace.
struct RouteDev {
  int32_t* hdr;
  RunPair* runs_src;   // ordered by zigzag row: out = zigzag row, in = token
  RunPair* runs_dst;   // ordered by token:      out = token,      in = zigzag row
  int32_t* split;      // [cp][cp]
  DirEntry* dir_src;   // entry for zigzag row 16*b (c->z output rows)
  DirEntry* dir_dst;   // entry for token 16*b (z->c output rows)
  int32_t* docs;       // compacted non-empty slots: [start | chunk | offset], docs_cap each
  int32_t docs_cap;
  int64_t run_cap;
};

// Launchers (return hipError_t of the launch).
// The whole build: runs, split matrix, header and directory (one launch, or
// a build launch followed by the directory launch for routes whose
// directory is too large to write from the build's workgroups).
hipError_t launch_route_build(const int32_t* cu, int32_t n_slots, int32_t cp, int32_t total,
                              const RouteDev& ws, hipStream_t stream);
hipError_t launch_route_index(const RouteDev& ws, int32_t total, hipStream_t stream);

// Swap launch overrides of one route; 0 in a field means the built-in choice.
struct SwapLaunch {
  int64_t tile_bytes;
  int32_t nontemporal;    // 1 on, 0 off
  int32_t block_threads;  // 128, 256, 512 or 1024
  int32_t tile_order;     // tiles per XCD chunk: 1 natural order, G > 1 XCD-chunked
};

// Plain streaming copy (thd_copy) in its own fixed shape.
hipError_t launch_copy(const void* in, void* out, int64_t bytes, hipStream_t stream);
hipError_t launch_read_stream(const void* in, int64_t bytes, const uint32_t key[4], uint32_t* count,
                              hipStream_t stream);
hipError_t launch_write_stream(void* out, int64_t bytes, uint32_t seed, hipStream_t stream);
// run_rows: the typical run length in rows the host expects (total rows over
// the 2 * cp * n_slots zigzag segments).  Rows of exactly one copy unit go
// through the LDS-staged small-row path when runs are shorter than one tile
// of the piecewise path, and through the piecewise path (a tile is then one
// or two flat copies) when they are at least that long.
hipError_t launch_swap(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir,
                       const void* in, void* out, int32_t total, int64_t row_bytes, int64_t run_rows,
                       const SwapLaunch& cfg, hipStream_t stream);

hipError_t launch_swap_batch(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir,
                             int32_t n, const void* const* ins, void* const* outs, const int64_t* row_bytes,
                             int32_t total, int64_t run_rows, hipStream_t stream);

// Token-order runs of a route, for writing the roll's outputs in zigzag order.
struct RollRoute {
  const int32_t* hdr;
  const RunPair* runs;
  const DirEntry* dir;
};

hipError_t launch_roll(const int64_t* ids, const int32_t* cu_pad, const int32_t* cu_real,
                       int32_t n_slots, int32_t total, int32_t max_shift, int64_t fill,
                       int64_t* shifted, uint8_t* mask, int32_t* status, const RollRoute* route,
                       hipStream_t stream);

// Views into the caller's packing workspace (see thd_pack_workspace_bytes).
struct PackWs {
  int32_t* hdr;           // [0] status, [1] documents, [2] padded tokens
  // per chunk of a row (batch-major), from the chunk pass
  int32_t* ch_lnp;        // last non-PAD position + 1 inside the chunk (row coordinates), 0: none
  int32_t* ch_ne;         // EOD tokens in the chunk
  int32_t* ch_fe;         // end (position + 1) of the chunk's first EOD, 0: none
  int32_t* ch_le;         // end of the chunk's last EOD, 0: none
  int64_t* ch_ps;         // padded lengths of the documents that start and end in the chunk
  // per chunk, from the scan pass
  int32_t* ch_prev;       // end of the last document of the row closed before the chunk
  int64_t* ch_doc_base;   // index of the first document that ends in or after the chunk
  int64_t* ch_pack_base;  // packed position where the document holding the chunk's first token starts
  // per row, from the scan pass
  int32_t* row_valid;     // valid end (last non-PAD position + 1)
  int64_t* row_real_off;  // valid tokens of the earlier rows
};

// Chunks the pack kernels cut a [batch, seq] batch into.
int64_t pack_chunks(int32_t batch, int32_t seq);

hipError_t launch_pack(const int64_t* tokens, int32_t batch, int32_t seq, int64_t pad_id, int64_t eod_id,
                       int32_t align, int32_t capacity, int32_t max_docs, int64_t pad_value, const PackWs& ws,
                       int64_t* packed, int32_t* cu_real, int32_t* cu_pad, int32_t* status, hipStream_t stream);

// Severity of a validation failure: larger wins; 0 = no failure.
__host__ __device__ inline int32_t severity_to_code(int sev) {
  switch (sev) {
    case 5: return THD_ERR_CU_START;
    case 4: return THD_ERR_CU_MONOTONE;
    case 3: return THD_ERR_CU_TOTAL;
    case 2: return THD_ERR_CU_DIVISIBLE;
    case 1: return THD_ERR_REAL_GT_PADDED;
    default: return THD_OK;
  }
}
constexpr int kSevStart = 5, kSevMonotone = 4, kSevTotal = 3, kSevDivisible = 2, kSevRealGtPadded = 1;

}  // namespace thdcp
