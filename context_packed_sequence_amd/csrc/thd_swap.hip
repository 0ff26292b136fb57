// Row permutation that applies a route: the single-GPU stand-in for the
// pack -> all-to-all -> scatter exchange of Relax PR #273 "fla mcore chunkwise
// cp stage 3", §2.1 (index_select into a send buffer, all_to_all, index_copy_
// out of the receive buffer).  With every rank's share in one emulated buffer,
// the three copies collapse into one: each output row is read once and
// written once.
//
// The route is a list of runs sorted by output row; inside a run both the
// input rows and the output rows are consecutive, so a run is one contiguous
// byte range on each side.  The output rows are cut into tiles of about
// 4 KiB per workgroup (whole rows, one row, or a slice of one long row); the
// route's directory entry for the tile's first row gives the input row, the
// end of its run, the run index and the run starts inside its 16-row block in
// one load.  A workgroup walks the runs that overlap its tile (almost always
// one) and streams each piece as a flat copy:
// consecutive lanes touch consecutive 16-byte vectors, so every wave-wide load
// and store is a fully coalesced 1 KiB access.  Run data is uniform across the
// workgroup and is read through scalar loads.
//
// The work is HBM-bound (2 * rows * row_bytes bytes, no arithmetic).  Many
// small workgroups keep the set of rows being copied at any moment inside a
// narrow, sliding address window, which is what lets a copy approach the HBM
// roofline; loads and stores are non-temporal because nothing is reused.
#include <climits>

#include "thd_device.h"
#include "thd_internal.h"

namespace thdcp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <bool NT, typename U>
__device__ __forceinline__ U load_unit(const U* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT, typename U>
__device__ __forceinline__ void store_unit(U* p, U v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <typename U, int BLOCK, int UNROLL, bool NT>
__device__ __forceinline__ void copy_span(const U* __restrict__ src, U* __restrict__ dst, int64_t n) {
  const int tid = threadIdx.x;
  int64_t base = 0;
  for (; base + BLOCK * UNROLL <= n; base += BLOCK * UNROLL) {
    U v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = load_unit<NT>(src + base + u * BLOCK + tid);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) store_unit<NT>(dst + base + u * BLOCK + tid, v[u]);
  }
  for (int64_t i = base + tid; i < n; i += BLOCK) store_unit<NT>(dst + i, load_unit<NT>(src + i));
}

// 16-byte output words from a source that is not 16-byte aligned: output
// word j (16-byte aligned) holds source bytes [s + 16 j, s + 16 j + 16) with
// s = a + 16 * D + B, a 16-byte aligned, D whole 4-byte words and B bytes
// (0 < 4 * D + B < 16).  The two aligned source words that cover those bytes
// are funnelled together, four 32-bit byte-aligns.  Both hold at least one
// byte of the source range, so no load leaves the pages the range lies in.
// Every lane of the workgroup must reach this call (BLOCK a multiple of 64):
// the lane shift reads the neighbour lane's registers.
template <int D, int BLOCK, int UNROLL, bool NT>
__device__ __forceinline__ void realign_words(const u32x4* __restrict__ a, u32x4* __restrict__ dst, int64_t n,
                                              uint32_t b) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  for (int64_t base = 0; base < n; base += BLOCK * UNROLL) {
    // lane l of a wave takes word j and needs source words j and j + 1; word
    // j + 1 is lane l + 1's first word, handed over by a DPP lane shift, so
    // only the wave's last lane and the range's last word load it themselves
    u32x4 lo[UNROLL], own_hi[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t j = base + u * BLOCK + tid;
      lo[u] = u32x4{0u, 0u, 0u, 0u};
      own_hi[u] = u32x4{0u, 0u, 0u, 0u};
      if (j < n) {
        lo[u] = load_unit<NT>(a + j);
        if (lane == 63 || j + 1 >= n) own_hi[u] = load_unit<NT>(a + j + 1);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t j = base + u * BLOCK + tid;
      // wave_shl:1: lane l reads lane l + 1; lane 63 keeps its own word
      const uint32_t h0 = __builtin_amdgcn_update_dpp(own_hi[u].x, lo[u].x, 0x130, 0xf, 0xf, false);
      const uint32_t h1 = __builtin_amdgcn_update_dpp(own_hi[u].y, lo[u].y, 0x130, 0xf, 0xf, false);
      const uint32_t h2 = __builtin_amdgcn_update_dpp(own_hi[u].z, lo[u].z, 0x130, 0xf, 0xf, false);
      const uint32_t h3 = __builtin_amdgcn_update_dpp(own_hi[u].w, lo[u].w, 0x130, 0xf, 0xf, false);
      // the last word of the range: its neighbour lane holds no source word
      const bool edge = lane == 63 || j + 1 >= n;
      const uint32_t w[8] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w,
                             edge ? own_hi[u].x : h0, edge ? own_hi[u].y : h1,
                             edge ? own_hi[u].z : h2, edge ? own_hi[u].w : h3};
      if (j < n) {
        u32x4 o;
        o.x = __builtin_amdgcn_alignbyte(w[D + 1], w[D], b);
        o.y = __builtin_amdgcn_alignbyte(w[D + 2], w[D + 1], b);
        o.z = __builtin_amdgcn_alignbyte(w[D + 3], w[D + 2], b);
        o.w = __builtin_amdgcn_alignbyte(w[D + 4], w[D + 3], b);
        store_unit<NT>(dst + j, o);
      }
    }
  }
}

// Bytes [src, src + n) to [dst, dst + n) for pointers and sizes that are
// multiples of sizeof(U) < 16: U-sized copies up to dst's first 16-byte
// boundary and after its last one, 16-byte stores in between whatever the
// source's alignment (a plain 16-byte copy when both sides share it).
template <typename U, int BLOCK, int PAIRS, bool NT>
__device__ __forceinline__ void copy_bytes_realigned(const unsigned char* __restrict__ src,
                                                     unsigned char* __restrict__ dst, int64_t n) {
  const int tid = threadIdx.x;
  const int64_t head = min(n, static_cast<int64_t>((16 - (reinterpret_cast<uintptr_t>(dst) & 15)) & 15));
  for (int64_t i = tid; i < head / static_cast<int64_t>(sizeof(U)); i += BLOCK)
    store_unit<NT>(reinterpret_cast<U*>(dst) + i, load_unit<NT>(reinterpret_cast<const U*>(src) + i));
  const int64_t words = (n - head) / 16;
  const unsigned char* s = src + head;
  u32x4* d = reinterpret_cast<u32x4*>(dst + head);
  const uint32_t m = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s) & 15);
  if (m == 0) {
    copy_span<u32x4, BLOCK, PAIRS, NT>(reinterpret_cast<const u32x4*>(s), d, words);
  } else {
    const u32x4* a = reinterpret_cast<const u32x4*>(s - m);
    switch (m >> 2) {
      case 0: realign_words<0, BLOCK, PAIRS, NT>(a, d, words, m & 3); break;
      case 1: realign_words<1, BLOCK, PAIRS, NT>(a, d, words, m & 3); break;
      case 2: realign_words<2, BLOCK, PAIRS, NT>(a, d, words, m & 3); break;
      default: realign_words<3, BLOCK, PAIRS, NT>(a, d, words, m & 3); break;
    }
  }
  const int64_t done = head + 16 * words;
  for (int64_t i = tid; i < (n - done) / static_cast<int64_t>(sizeof(U)); i += BLOCK)
    store_unit<NT>(reinterpret_cast<U*>(dst + done) + i, load_unit<NT>(reinterpret_cast<const U*>(src + done) + i));
}

// Pieces of at least this many bytes in units under 16 bytes go through the
// realigning copy.
constexpr int64_t kRealignMinBytes = 256;

// One tile of output rows [r0, r1): find the run holding r0 from e, the
// directory entry of r0's 16-row block (it alone covers the usual case where
// no run starts between the block's first row and r0; otherwise the entry's
// run-start bits name the run, and one load of it follows), then copy run
// piece by run piece.  Every access stays inside the run table and inside
// [0, total) rows of both buffers.
// PAIRS: source-word pairs in flight per thread in the realigning copy (two
// source words per output word, so half a plain copy's unroll keeps the
// registers in flight the same); 0 leaves narrow units to the plain copy.
template <typename U, int BLOCK, int UNROLL, bool NT, int PAIRS = (UNROLL > 2 ? UNROLL / 2 : 1)>
__device__ __forceinline__ void swap_tile(const RunPair* __restrict__ runs, const DirEntry& e, int32_t n_runs,
                                          const unsigned char* __restrict__ in, unsigned char* __restrict__ out,
                                          int32_t total, int64_t row_bytes, int32_t r0, int32_t r1) {
  int32_t k, in_row, run_end;
  if (r0 < e.run_end) {
    k = e.run;
    in_row = e.in + (r0 & (kDirBlock - 1));
    run_end = e.run_end;
  } else {
    k = run_of_row(e, r0);
    if (k >= n_runs) return;
    const RunPair run = runs[k];
    if (run.out > r0) return;
    in_row = run.in + (r0 - run.out);
    run_end = (k + 1 < n_runs) ? runs[k + 1].out : total;
  }
  while (true) {
    const int32_t piece_end = min(r1, run_end);
    const U* src = reinterpret_cast<const U*>(in + static_cast<int64_t>(in_row) * row_bytes);
    U* dst = reinterpret_cast<U*>(out + static_cast<int64_t>(r0) * row_bytes);
    const int64_t n_units = static_cast<int64_t>(piece_end - r0) * row_bytes / static_cast<int64_t>(sizeof(U));
    if constexpr (sizeof(U) < 16 && PAIRS > 0) {
      if (n_units * static_cast<int64_t>(sizeof(U)) >= kRealignMinBytes)
        copy_bytes_realigned<U, BLOCK, PAIRS, NT>(reinterpret_cast<const unsigned char*>(src),
                                                   reinterpret_cast<unsigned char*>(dst),
                                                   n_units * static_cast<int64_t>(sizeof(U)));
      else
        copy_span<U, BLOCK, UNROLL, NT>(src, dst, n_units);
    } else {
      copy_span<U, BLOCK, UNROLL, NT>(src, dst, n_units);
    }
    r0 = piece_end;
    if (r0 >= r1 || ++k >= n_runs) break;
    const RunPair run = runs[k];
    if (run.out != r0) break;  // runs tile the output rows; never trust anything else
    in_row = run.in;
    run_end = (k + 1 < n_runs) ? runs[k + 1].out : total;
  }
}

// Part of one output row: bytes [b0, b1) of row r, for rows so long that a
// workgroup takes a slice of a row rather than whole rows; e is the directory
// entry of r's 16-row block.
template <typename U, int BLOCK, int UNROLL, bool NT>
__device__ __forceinline__ void swap_row_part(const RunPair* __restrict__ runs, const DirEntry& e, int32_t n_runs,
                                              const unsigned char* __restrict__ in, unsigned char* __restrict__ out,
                                              int64_t row_bytes, int32_t r, int64_t b0, int64_t b1) {
  int32_t in_row;
  if (r < e.run_end) {
    in_row = e.in + (r & (kDirBlock - 1));
  } else {
    const int32_t k = run_of_row(e, r);
    if (k >= n_runs) return;
    const RunPair run = runs[k];
    if (run.out > r) return;
    in_row = run.in + (r - run.out);
  }
  const U* src = reinterpret_cast<const U*>(in + static_cast<int64_t>(in_row) * row_bytes + b0);
  U* dst = reinterpret_cast<U*>(out + static_cast<int64_t>(r) * row_bytes + b0);
  copy_span<U, BLOCK, UNROLL, NT>(src, dst, (b1 - b0) / static_cast<int64_t>(sizeof(U)));
}

// Small rows (row_bytes equal to the copy unit, at most 16 B: token ids,
// labels, masks, position ids): copying run piece by run piece would leave
// most lanes idle on short pieces, so the tile's runs are staged in LDS and
// every thread looks up the run of each of its rows there, then moves the
// row with one load and one store.  Consecutive lanes take consecutive
// output rows, so the stores are fully coalesced, and so are the loads inside
// a run.  Tiles whose rows cross more than kSmallStage runs fall back to the
// piecewise copy.
constexpr int kSmallRowsPerThread = 4;
constexpr int kSmallStage = 512;

template <typename U, int BLOCK, bool NT>
__device__ __forceinline__ void swap_tile_small(const RunPair* __restrict__ runs, const DirEntry* __restrict__ dir,
                                                int32_t n_runs, const unsigned char* __restrict__ in8,
                                                unsigned char* __restrict__ out8, int32_t total, int32_t r0,
                                                int32_t r1, RunPair* s_runs, int32_t* s_k) {
  const int tid = threadIdx.x;
  if (tid < 2) {  // run holding the first row and run holding the last row of the tile
    const int32_t row = tid == 0 ? r0 : r1 - 1;
    const DirEntry e = dir[row >> kDirShift];
    const int32_t k = row < e.run_end ? e.run : run_of_row(e, row);
    s_k[tid] = min(k, n_runs - 1);
  }
  __syncthreads();
  const int32_t k0 = s_k[0];
  const int32_t cnt = s_k[1] - k0 + 1;
  if (cnt <= kSmallStage) {
    for (int i = tid; i < cnt; i += BLOCK) s_runs[i] = runs[k0 + i];
    __syncthreads();
    const U* in = reinterpret_cast<const U*>(in8);
    U* out = reinterpret_cast<U*>(out8);
    U v[kSmallRowsPerThread];
#pragma unroll
    for (int m = 0; m < kSmallRowsPerThread; ++m) {
      const int32_t r = r0 + m * BLOCK + tid;
      if (r < r1) {
        int32_t lo = 0, hi = cnt;  // s_runs[lo].out <= r
        while (hi - lo > 1) {
          const int32_t mid = (lo + hi) >> 1;
          if (s_runs[mid].out <= r) lo = mid;
          else hi = mid;
        }
        v[m] = load_unit<NT>(in + (s_runs[lo].in + (r - s_runs[lo].out)));
      }
    }
#pragma unroll
    for (int m = 0; m < kSmallRowsPerThread; ++m) {
      const int32_t r = r0 + m * BLOCK + tid;
      if (r < r1) store_unit<NT>(out + r, v[m]);
    }
  } else {
    swap_tile<U, BLOCK, 8, NT, 0>(runs, dir[r0 >> kDirShift], n_runs, in8, out8, total,
                                  static_cast<int64_t>(sizeof(U)), r0, r1);
  }
  __syncthreads();  // the next tile reuses s_runs and s_k
}

template <typename U, int BLOCK, bool NT>
__global__ __launch_bounds__(BLOCK) void swap_small_kernel(const int32_t* __restrict__ hdr, int runs_word,
                                                           const RunPair* __restrict__ runs,
                                                           const DirEntry* __restrict__ dir,
                                                           const unsigned char* __restrict__ in,
                                                           unsigned char* __restrict__ out, int32_t total,
                                                           int32_t n_tiles) {
  __shared__ RunPair s_runs[kSmallStage];
  __shared__ int32_t s_k[2];
  if (hdr[kHdrStatus] != THD_OK) return;
  const int32_t n_runs = hdr[runs_word];
  constexpr int32_t kTileRows = BLOCK * kSmallRowsPerThread;
  for (int32_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int32_t r0 = static_cast<int32_t>(static_cast<int64_t>(tile) * kTileRows);
    const int32_t r1 = static_cast<int32_t>(min(static_cast<int64_t>(total), static_cast<int64_t>(r0) + kTileRows));
    swap_tile_small<U, BLOCK, NT>(runs, dir, n_runs, in, out, total, r0, r1, s_runs, s_k);
  }
}

// Tile order.  The chip hands workgroup b to XCD b mod 8.  Natural order
// (chunk 1): workgroup b copies tile b, so consecutive tiles land on
// different XCDs.  XCD-chunked order (chunk G): the tiles are cut into chunks
// of G, XCD x takes chunks x, x + 8, x + 16, ... and walks each chunk front to
// back, i.e. workgroup b = 8 j + x copies tile ((j / G) * 8 + x) * G + j mod G.
constexpr int kXcds = 8;

__device__ __forceinline__ int32_t tile_of_slot(int32_t slot, int32_t chunk) {
  const int32_t x = slot % kXcds, j = slot / kXcds;
  return chunk == 1 ? slot : ((j / chunk) * kXcds + x) * chunk + j % chunk;
}

// One tile per workgroup.  Capped at 64 VGPRs (8 waves per SIMD); the
// 16-byte-unit kernels need under 50, the narrow ones 63-64 with no spills.
//
// A workgroup lives a few microseconds and moves a few KiB, so the memory
// round trips before its first data load are a visible share of its life.
// The route's status word, its run count and the directory entry of the
// tile's first row do not depend on each other and are read in one round
// trip: the empty asm statement takes all three as operands before the
// status test, so no load can sink below the test.  The entry's address lies
// inside the directory whatever the status; its value is used only once the
// status is good.  (Measured on MI355X: 0.6-1.2 % on 4 KiB rows against
// reading the status first.  The same reads inside a loop over several tiles
// per workgroup cost 5 %, so the kernel takes exactly one.)
template <typename U, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(8))) void swap_kernel(const int32_t* __restrict__ hdr, int runs_word,
                                                     const RunPair* __restrict__ runs,
                                                     const DirEntry* __restrict__ dir,
                                                     const unsigned char* __restrict__ in,
                                                     unsigned char* __restrict__ out, int32_t total,
                                                     int64_t row_bytes, int32_t tile_rows, int32_t n_tiles,
                                                     int32_t chunk, int32_t parts, int64_t part_bytes) {
  const int32_t tile = tile_of_slot(blockIdx.x, chunk);
  if (tile >= n_tiles) return;
  // first output row of the tile (rows cut into slices: tile = (row, slice))
  const int32_t r = parts > 1 ? tile / parts : tile * tile_rows;
  const int32_t status = hdr[kHdrStatus];
  const int32_t n_runs = hdr[runs_word];
  const DirEntry e = dir[r >> kDirShift];
  asm volatile("" ::"s"(status), "s"(n_runs), "s"(e.in), "s"(e.run_end), "s"(e.run), "s"(e.starts));
  if (status != THD_OK) return;  // a failed build writes nothing
  if (parts > 1) {
    const int64_t b0 = static_cast<int64_t>(tile - r * parts) * part_bytes;
    swap_row_part<U, BLOCK, UNROLL, NT>(runs, e, n_runs, in, out, row_bytes, r, b0, min(row_bytes, b0 + part_bytes));
  } else {
    const int32_t r1 = static_cast<int32_t>(min(static_cast<int64_t>(total), static_cast<int64_t>(r) + tile_rows));
    swap_tile<U, BLOCK, UNROLL, NT>(runs, e, n_runs, in, out, total, row_bytes, r, r1);
  }
}

// Several tensors through one route in one launch (the tokens, labels,
// loss mask, position ids and valid mask of a batch, or the projections of one
// layer): the launch's tiles are the concatenation of every tensor's tiles,
// each tensor with its own row size and copy unit.
struct BatchTensor {
  const unsigned char* in;
  unsigned char* out;
  int64_t row_bytes;
  int32_t tile_rows;
  int32_t first_tile;  // index of the tensor's first tile in the launch
  int32_t unit;        // copy unit in bytes: 16, 8, 4, 2 or 1
  int32_t parts;       // > 1: each tile is one part of one row, part_bytes long
  int64_t part_bytes;
  int32_t small;       // one-unit rows of 1-8 B with short runs: the LDS-staged path
};

struct BatchArgs {
  BatchTensor t[THD_MAX_BATCH];
  int32_t n;
  int32_t total_tiles;
  int32_t chunk;    // tiles per XCD chunk (1: natural order), as in swap_kernel
};

constexpr int kBatchBlock = 128;

// One tile per workgroup; the tile's tensor is found in the kernel arguments,
// then the route status, run count and directory entry of the tile's first
// row are read in one round trip, as in swap_kernel.
__global__ __launch_bounds__(kBatchBlock) __attribute__((amdgpu_waves_per_eu(8))) void swap_batch_kernel(const int32_t* __restrict__ hdr, int runs_word,
                                                                 const RunPair* __restrict__ runs,
                                                                 const DirEntry* __restrict__ dir, int32_t total,
                                                                 BatchArgs args) {
  __shared__ RunPair s_runs[kSmallStage];
  __shared__ int32_t s_k[2];
  const int32_t g = tile_of_slot(blockIdx.x, args.chunk);
  if (g >= args.total_tiles) return;
  int i = 0;
  while (i + 1 < args.n && args.t[i + 1].first_tile <= g) ++i;
  const BatchTensor bt = args.t[i];
  // first output row of the tile (long rows: tile = (row, slice))
  const int32_t r = bt.parts > 1 ? (g - bt.first_tile) / bt.parts
                                 : static_cast<int32_t>(static_cast<int64_t>(g - bt.first_tile) * bt.tile_rows);
  const int32_t status = hdr[kHdrStatus];
  const int32_t n_runs = hdr[runs_word];
  const DirEntry e = dir[r >> kDirShift];
  asm volatile("" ::"s"(status), "s"(n_runs), "s"(e.in), "s"(e.run_end), "s"(e.run), "s"(e.starts));
  if (status != THD_OK) return;  // a failed build writes nothing
  if (bt.parts > 1) {  // long rows (16-byte units only): one slice of one row per tile
    const int64_t b0 = static_cast<int64_t>((g - bt.first_tile) % bt.parts) * bt.part_bytes;
    const int64_t b1 = min(bt.row_bytes, b0 + bt.part_bytes);
    swap_row_part<u32x4, kBatchBlock, 8, true>(runs, e, n_runs, bt.in, bt.out, bt.row_bytes, r, b0, b1);
    return;
  }
  const int32_t r1 = static_cast<int32_t>(min(static_cast<int64_t>(total), static_cast<int64_t>(r) + bt.tile_rows));
  if (bt.small) {  // one unit per row, short runs: the LDS-staged small-row path
    switch (bt.unit) {
      case 8: swap_tile_small<u32x2, kBatchBlock, true>(runs, dir, n_runs, bt.in, bt.out, total, r, r1, s_runs, s_k); break;
      case 4: swap_tile_small<uint32_t, kBatchBlock, true>(runs, dir, n_runs, bt.in, bt.out, total, r, r1, s_runs, s_k); break;
      case 2: swap_tile_small<uint16_t, kBatchBlock, true>(runs, dir, n_runs, bt.in, bt.out, total, r, r1, s_runs, s_k); break;
      default: swap_tile_small<uint8_t, kBatchBlock, true>(runs, dir, n_runs, bt.in, bt.out, total, r, r1, s_runs, s_k); break;
    }
    return;
  }
  switch (bt.unit) {
    case 16: swap_tile<u32x4, kBatchBlock, 8, true>(runs, e, n_runs, bt.in, bt.out, total, bt.row_bytes, r, r1); break;
    case 8: swap_tile<u32x2, kBatchBlock, 8, true>(runs, e, n_runs, bt.in, bt.out, total, bt.row_bytes, r, r1); break;
    case 4: swap_tile<uint32_t, kBatchBlock, 8, true>(runs, e, n_runs, bt.in, bt.out, total, bt.row_bytes, r, r1); break;
    case 2: swap_tile<uint16_t, kBatchBlock, 8, true>(runs, e, n_runs, bt.in, bt.out, total, bt.row_bytes, r, r1); break;
    default: swap_tile<uint8_t, kBatchBlock, 8, true>(runs, e, n_runs, bt.in, bt.out, total, bt.row_bytes, r, r1); break;
  }
}

// Plain streaming copy of 4 KiB tiles: no route, no permutation.  The swap's
// units, tiles and non-temporal loads, in XCD-chunked order with chunks of
// 256 tiles.  16-byte units: 256 threads, one word per lane, and a tile that
// covers whole 128-byte lines stores through StreamStore (write-through):
// the fastest plain copy in sweeps on MI355X, 2.5-4 % ahead of the same
// copy with non-temporal stores and 0.8-3 % ahead of 128 threads with two
// words per lane and non-temporal stores.
// (The swap keeps non-temporal stores: its permuted reads already run it at
// this copy's speed, and write-through stores gained it nothing.)
template <typename U, int BLOCK, int UNROLL>
__global__ __launch_bounds__(BLOCK) void copy_kernel(const unsigned char* __restrict__ in,
                                                     unsigned char* __restrict__ out, int64_t bytes,
                                                     int64_t tile_bytes, int32_t n_tiles, int32_t chunk) {
  const int32_t tile = tile_of_slot(blockIdx.x, chunk);
  if (tile >= n_tiles) return;
  const int64_t b0 = static_cast<int64_t>(tile) * tile_bytes;
  const int64_t n = min(tile_bytes, bytes - b0) / static_cast<int64_t>(sizeof(U));
  const U* src = reinterpret_cast<const U*>(in + b0);
  U* dst = reinterpret_cast<U*>(out + b0);
  if constexpr (sizeof(U) == 16) {
    const int32_t bytes_here = static_cast<int32_t>(n) * 16;
    if (((reinterpret_cast<uintptr_t>(dst) | static_cast<uintptr_t>(bytes_here)) & 127) == 0) {
      const StreamStore st(dst, bytes_here);
      for (int32_t i = threadIdx.x; i < n; i += BLOCK) st(i, __builtin_nontemporal_load(src + i));
      return;
    }
  }
  copy_span<U, BLOCK, UNROLL, true>(src, dst, n);
}

// Whole-row tile of about tile_bytes whose byte length is a multiple of 128
// (a whole number of cache lines), so neighbouring tiles never write parts
// of one line; rows for which no such tile fits in tile_bytes keep the plain
// rounding.  Measured: 4-13 % on rows of 3-100 bytes that are not powers of
// two.
int64_t whole_row_tile(int64_t row_bytes, int64_t tile_bytes) {
  int64_t g = 128, r = row_bytes;
  while (r) {
    const int64_t t = g % r;
    g = r;
    r = t;
  }
  const int64_t q = 128 / g;  // rows per 128-byte multiple
  if (q * row_bytes > tile_bytes) return (tile_bytes + row_bytes - 1) / row_bytes;
  return tile_bytes / row_bytes / q * q;
}

// A dispatch counts its work-items in 32 bits: a launch past that is refused
// on the host rather than handed to the runtime.
bool fits_dispatch(int64_t workgroups, int64_t threads) { return workgroups * threads <= static_cast<int64_t>(UINT32_MAX); }

int copy_unit(int64_t row_bytes, const void* in, const void* out) {
  const uint64_t align_bits = static_cast<uint64_t>(row_bytes) | reinterpret_cast<uintptr_t>(in) |
                              reinterpret_cast<uintptr_t>(out);
  int unit = 16;
  while (unit > 1 && (align_bits & (unit - 1))) unit >>= 1;
  return unit;
}

struct Shape {
  int32_t tile_rows, n_tiles, chunk, grid, parts;
  int64_t part_bytes;
};

template <typename U, int BLOCK, int UNROLL>
hipError_t launch_typed(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir, const void* in,
                        void* out, int32_t total, int64_t row_bytes, const Shape& sh, bool nt, hipStream_t stream) {
  const auto* i8 = static_cast<const unsigned char*>(in);
  auto* o8 = static_cast<unsigned char*>(out);
  if (nt)
    hipLaunchKernelGGL((swap_kernel<U, BLOCK, UNROLL, true>), dim3(sh.grid), dim3(BLOCK), 0, stream, hdr, runs_word,
                       runs, dir, i8, o8, total, row_bytes, sh.tile_rows, sh.n_tiles, sh.chunk, sh.parts,
                       sh.part_bytes);
  else
    hipLaunchKernelGGL((swap_kernel<U, BLOCK, UNROLL, false>), dim3(sh.grid), dim3(BLOCK), 0, stream, hdr, runs_word,
                       runs, dir, i8, o8, total, row_bytes, sh.tile_rows, sh.n_tiles, sh.chunk, sh.parts,
                       sh.part_bytes);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swap(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir, const void* in,
                       void* out, int32_t total, int64_t row_bytes, int64_t run_rows, const SwapLaunch& cfg,
                       hipStream_t stream) {
  // Widest unit that divides the row size and both base addresses.
  const int unit = copy_unit(row_bytes, in, out);

  // Tile of the piecewise path for units under 16 bytes: 8 KiB (sweeps of
  // 1-100-byte rows on 1 GiB swaps, with the realigning copy).
  const int64_t unit_tile_bytes = 8192;

  // One-unit rows: the LDS-staged path when runs are shorter than a tile of
  // the piecewise path; with longer runs the piecewise path streams them as
  // flat copies, 5-300 % faster on batches of 256 MiB and more.
  const int64_t flat_tile_rows = (unit == 16 ? 4096 : unit_tile_bytes) / unit;
  if (row_bytes == unit && cfg.tile_bytes == 0 && cfg.block_threads == 0 && run_rows < flat_tile_rows) {
    constexpr int kBlock = 256;
    const int64_t tiles = (static_cast<int64_t>(total) + kBlock * kSmallRowsPerThread - 1) /
                          (kBlock * kSmallRowsPerThread);
    if (!fits_dispatch(tiles, kBlock)) return hipErrorInvalidValue;
    const int32_t grid = static_cast<int32_t>(tiles);
    if (grid <= 0) return hipSuccess;
    const auto* i8 = static_cast<const unsigned char*>(in);
    auto* o8 = static_cast<unsigned char*>(out);
    const int32_t nt_ = static_cast<int32_t>(tiles);
#define THD_SMALL(U_)                                                                                               \
  hipLaunchKernelGGL((swap_small_kernel<U_, kBlock, true>), dim3(grid), dim3(kBlock), 0, stream, hdr, runs_word, runs, \
                     dir, i8, o8, total, nt_)
    switch (unit) {
      case 16: THD_SMALL(u32x4); break;
      case 8: THD_SMALL(u32x2); break;
      case 4: THD_SMALL(uint32_t); break;
      case 2: THD_SMALL(uint16_t); break;
      default: THD_SMALL(uint8_t); break;
    }
#undef THD_SMALL
    return hipGetLastError();
  }

  // Launch shape, measured on MI355X (interleaved sweeps on one box, 1 GiB
  // per swap, after a warm-up).  Rows moved in 16-byte units run fastest when
  // every 256-thread workgroup moves 4-6 KiB, one or at most one and a half
  // 16-byte words per lane:
  //  * rows of whole 4 KiB pages (4, 8, 12, 16 KiB, ...): one 4 KiB slice of
  //    a row per workgroup, one word per lane, XCD-chunked order with chunks
  //    of 256 tiles (8-16 KiB rows 1.2-1.5 % faster than 4 KiB slices on 128
  //    threads with two words per lane);
  //  * other rows above 4 KiB (5120, 6144, 10240, ...): slices of 4-6 KiB,
  //    chunks of 64 (5120- and 6144-byte rows 2-3 % faster than one row per
  //    workgroup in chunks of 256);
  //  * rows between 1 and 4 KiB that are not powers of two: as many whole
  //    rows as fit in 6 KiB per workgroup, chunks of 64 (4000-byte rows 6 %,
  //    2560- and 3072-byte rows 1-2 % faster than the earlier shapes);
  //  * shorter rows, and 1 KiB and 2 KiB rows: the most whole rows that fit
  //    in 4 KiB on 256 threads, XCD-chunked order with chunks of 256 tiles
  //    (64 for rows under 64 bytes), when those rows hold at least 220
  //    16-byte words: against 128 threads in natural order with tiles of
  //    whole 128-byte lines, 0.6-1.4 % faster on 64-2048-byte rows, 2-13 %
  //    on rows that are not powers of two (272-byte rows 188.5 -> 163.7 us
  //    per GiB swap), level on 16- and 32-byte rows; rows whose 4 KiB tile
  //    would hold fewer words keep the whole-line tile (below).
  // Units under 16 bytes: 256 threads, 8 KiB tiles, chunks of 64.  Every
  // field can be overridden per route for sweeps; a tile size below the row
  // size cuts rows into slices.
  const bool pow2 = (row_bytes & (row_bytes - 1)) == 0;
  const bool page_rows = unit == 16 && row_bytes % 4096 == 0;
  const bool wide_rows = unit == 16 && row_bytes > 4096 && !page_rows;
  const bool kib_rows = unit == 16 && row_bytes > 1024 && row_bytes < 4096 && !pow2;
  const bool shaped = page_rows || wide_rows || kib_rows;
  int64_t auto_tile = unit == 16 ? 4096 : unit_tile_bytes;
  if (wide_rows) {
    const int64_t parts = (row_bytes + 6143) / 6144;
    auto_tile = (row_bytes + parts - 1) / parts;
  } else if (kib_rows) {
    auto_tile = (6144 / row_bytes) * row_bytes;
  }
  const int64_t tile_bytes = cfg.tile_bytes > 0 ? cfg.tile_bytes : auto_tile;
  int64_t tile_rows = cfg.tile_bytes == 0 && !shaped ? whole_row_tile(row_bytes, tile_bytes)
                                                     : (tile_bytes + row_bytes - 1) / row_bytes;
  if (tile_rows < 1) tile_rows = 1;
  if (tile_rows > (1 << 30)) tile_rows = 1 << 30;
  // 16-byte rows under 4 KiB: as many whole rows as fit in 4 KiB when they
  // fill at least 220 of the 256 lanes' 16-byte words (on 256 threads, up to
  // 13 % faster than the tile of whole 128-byte lines when that one fills
  // fewer); otherwise the whole-line tile, on 256 threads in XCD-chunked
  // order when it fills at least 240 words, else on 128 threads in natural
  // order (832-byte rows: 3328-byte tiles, 2.4 % slower on 256 threads).
  bool full_tile = false;
  if (cfg.tile_bytes == 0 && unit == 16 && !shaped) {
    const int64_t most = 4096 / row_bytes;
    if (most >= 1 && most * row_bytes >= 220 * 16) {
      tile_rows = most;
      full_tile = true;
    }
  }
  full_tile = full_tile || tile_rows * row_bytes >= 240 * 16;
  int block = cfg.block_threads > 0 ? cfg.block_threads : (unit == 16 && !shaped && !full_tile ? 128 : 256);
  int64_t chunk = cfg.tile_order > 0 ? cfg.tile_order
                  : page_rows        ? 256
                  : shaped           ? 64
                  : unit != 16       ? 64
                  : !full_tile       ? 1
                  : row_bytes >= 64  ? 256
                                     : 64;
  Shape sh;
  sh.tile_rows = static_cast<int32_t>(tile_rows);
  sh.parts = 1;
  sh.part_bytes = row_bytes;
  int64_t n_tiles = (total + tile_rows - 1) / tile_rows;
  if (unit == 16 && tile_bytes < row_bytes) {  // tiles are slices of one row
    int64_t parts = (row_bytes + tile_bytes - 1) / tile_bytes;
    // slices of whole 128-byte lines when the row is made of whole lines
    const int64_t grain = row_bytes % 128 == 0 ? 128 : 16;
    sh.part_bytes = ((row_bytes + parts - 1) / parts + grain - 1) / grain * grain;
    parts = (row_bytes + sh.part_bytes - 1) / sh.part_bytes;
    n_tiles = static_cast<int64_t>(total) * parts;
    if (parts > INT32_MAX || n_tiles > INT32_MAX) return hipErrorInvalidValue;
    sh.parts = static_cast<int32_t>(parts);
  }
  sh.n_tiles = static_cast<int32_t>(n_tiles);
  const int64_t per_xcd = (sh.n_tiles + kXcds - 1) / kXcds;
  if (chunk > per_xcd) chunk = per_xcd > 0 ? per_xcd : 1;  // one chunk per XCD at most
  sh.chunk = static_cast<int32_t>(chunk);
  const int64_t slots = chunk == 1 ? sh.n_tiles : (sh.n_tiles + kXcds * chunk - 1) / (kXcds * chunk) * kXcds * chunk;
  if (slots > INT32_MAX) return hipErrorInvalidValue;
  sh.grid = static_cast<int32_t>(slots);
  if (sh.grid <= 0) return hipSuccess;
  // a built-in block size whose grid would pass 2^32 work-items (tiles of a
  // few rows, set by an override) drops to 128 threads per workgroup
  if (cfg.block_threads == 0 && unit == 16 && !fits_dispatch(sh.grid, block)) block = 128;
  if (!fits_dispatch(sh.grid, unit == 16 ? block : 256)) return hipErrorInvalidValue;
  const bool nt = cfg.nontemporal != 0;
#define THD_SWAP_ARGS hdr, runs, runs_word, dir, in, out, total, row_bytes, sh, nt, stream
  switch (unit) {
    case 16:
      switch (block) {
        case 128: return launch_typed<u32x4, 128, 8>(THD_SWAP_ARGS);
        case 512: return launch_typed<u32x4, 512, 2>(THD_SWAP_ARGS);
        case 1024: return launch_typed<u32x4, 1024, 2>(THD_SWAP_ARGS);
        default: return launch_typed<u32x4, 256, 4>(THD_SWAP_ARGS);
      }
    case 8: return launch_typed<u32x2, 256, 8>(THD_SWAP_ARGS);
    case 4: return launch_typed<uint32_t, 256, 8>(THD_SWAP_ARGS);
    case 2: return launch_typed<uint16_t, 256, 8>(THD_SWAP_ARGS);
    default: return launch_typed<uint8_t, 256, 8>(THD_SWAP_ARGS);
  }
#undef THD_SWAP_ARGS
}

hipError_t launch_swap_batch(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir,
                             int32_t n, const void* const* ins, void* const* outs, const int64_t* row_bytes,
                             int32_t total, int64_t run_rows, hipStream_t stream) {
  BatchArgs args{};
  args.n = n;
  int64_t tiles = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int unit = copy_unit(row_bytes[i], ins[i], outs[i]);
    const int64_t tile_bytes = unit == 16 ? 4096 : 8192;
    // one-unit rows of 1-8 B with runs shorter than a piecewise tile: the
    // LDS-staged path, as for thd_swap
    const bool small = row_bytes[i] == unit && unit < 16 && run_rows < tile_bytes / unit;
    int64_t tile_rows = small                       ? kBatchBlock * kSmallRowsPerThread
                        : row_bytes[i] <= tile_bytes ? whole_row_tile(row_bytes[i], tile_bytes)
                                                     : (tile_bytes + row_bytes[i] - 1) / row_bytes[i];
    if (tile_rows < 1) tile_rows = 1;
    if (tile_rows > (1 << 30)) tile_rows = 1 << 30;
    // rows longer than a tile (16-byte units): every workgroup still moves
    // about 4 KiB, a slice of one row
    int64_t parts = 1, part_bytes = row_bytes[i];
    if (unit == 16 && row_bytes[i] > tile_bytes) {
      parts = (row_bytes[i] + tile_bytes - 1) / tile_bytes;
      const int64_t grain = row_bytes[i] % 128 == 0 ? 128 : 16;  // whole lines where the row has them
      part_bytes = ((row_bytes[i] + parts - 1) / parts + grain - 1) / grain * grain;
      parts = (row_bytes[i] + part_bytes - 1) / part_bytes;
      if (parts > INT32_MAX) return hipErrorInvalidValue;
    }
    args.t[i].in = static_cast<const unsigned char*>(ins[i]);
    args.t[i].out = static_cast<unsigned char*>(outs[i]);
    args.t[i].row_bytes = row_bytes[i];
    args.t[i].tile_rows = static_cast<int32_t>(tile_rows);
    args.t[i].first_tile = static_cast<int32_t>(tiles);
    args.t[i].unit = unit;
    args.t[i].parts = static_cast<int32_t>(parts);
    args.t[i].part_bytes = part_bytes;
    args.t[i].small = small ? 1 : 0;
    tiles += parts > 1 ? static_cast<int64_t>(total) * parts : (total + tile_rows - 1) / tile_rows;
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
  }
  if (tiles <= 0) return hipSuccess;
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  args.total_tiles = static_cast<int32_t>(tiles);
  // XCD-chunked tile order (chunks of 64 tiles of about 4 KiB), as the
  // single-tensor swap uses for long rows
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
  args.chunk = static_cast<int32_t>(per_xcd < 64 ? per_xcd : 64);
  const int64_t slots = args.chunk == 1 ? tiles : (tiles + kXcds * args.chunk - 1) / (kXcds * args.chunk) * kXcds * args.chunk;
  if (slots > INT32_MAX) return hipErrorInvalidValue;
  if (!fits_dispatch(slots, kBatchBlock)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(swap_batch_kernel, dim3(static_cast<unsigned>(slots)), dim3(kBatchBlock), 0, stream, hdr,
                     runs_word, runs, dir, total, args);
  return hipGetLastError();
}

hipError_t launch_copy(const void* in, void* out, int64_t bytes, hipStream_t stream) {
  const int unit = copy_unit(bytes, in, out);
  const int64_t tile_bytes = unit == 16 ? 4096 : 8192;
  const int64_t tiles = (bytes + tile_bytes - 1) / tile_bytes;
  if (tiles <= 0) return hipSuccess;
  if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
  const int32_t n_tiles = static_cast<int32_t>(tiles);
  int32_t chunk = unit == 16 ? 256 : 1;
  const int32_t per_xcd = (n_tiles + kXcds - 1) / kXcds;
  if (chunk > per_xcd) chunk = per_xcd;
  const int64_t slots =
      chunk == 1 ? n_tiles : (static_cast<int64_t>(n_tiles) + kXcds * chunk - 1) / (kXcds * chunk) * kXcds * chunk;
  if (slots > INT32_MAX || !fits_dispatch(slots, 256)) return hipErrorInvalidValue;
  const auto* i8 = static_cast<const unsigned char*>(in);
  auto* o8 = static_cast<unsigned char*>(out);
  const dim3 grid(static_cast<unsigned>(slots));
#define THD_COPY(U_, B_, R_) \
  hipLaunchKernelGGL((copy_kernel<U_, B_, R_>), grid, dim3(B_), 0, stream, i8, o8, bytes, tile_bytes, n_tiles, chunk)
  switch (unit) {
    case 16: THD_COPY(u32x4, 256, 1); break;
    case 8: THD_COPY(u32x2, 256, 4); break;
    case 4: THD_COPY(uint32_t, 256, 8); break;
    case 2: THD_COPY(uint16_t, 256, 8); break;
    default: THD_COPY(uint8_t, 256, 8); break;
  }
#undef THD_COPY
  return hipGetLastError();
}

}  // namespace thdcp
