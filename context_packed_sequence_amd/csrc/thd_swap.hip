// Row permutation that applies a route: the single-GPU stand-in for the
// pack -> all-to-all -> scatter exchange of Relax PR #273 "fla mcore chunkwise
// cp stage 3", §2.1 (index_select into a send buffer, all_to_all, index_copy_
// out of the receive buffer).  With every rank's share in one emulated buffer,
// the three copies collapse into one: each output row is read once and
// written once.
//
// The route is a list of runs sorted by output row; inside a run both the
// input rows and the output rows are consecutive, so a run is one contiguous
// byte range on each side.  The output rows are cut into tiles of whole rows
// (about one row, or 4 KiB of small rows, per workgroup); the route's
// directory entry for the tile's first row gives the input row, the end of its
// run and the run index in one load.  A workgroup walks the runs that overlap
// its tile (almost always one) and streams each piece as a flat copy:
// consecutive lanes touch consecutive 16-byte vectors, so every wave-wide load
// and store is a fully coalesced 1 KiB access.  Run data is uniform across the
// workgroup and is read through scalar loads.
//
// The work is HBM-bound (2 * rows * row_bytes bytes, no arithmetic).  Many
// small workgroups keep the set of rows being copied at any moment inside a
// narrow, sliding address window, which is what lets a copy approach the HBM
// roofline; loads and stores are non-temporal because nothing is reused.
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

// Tile order.  Natural: workgroup b copies tile b.  XCD-grouped: the chip
// hands workgroup b to XCD b mod 8, so tile (b mod 8) * ceil(n/8) + b / 8 gives
// every XCD one contiguous eighth of the output, streamed front to back.
constexpr int kXcds = 8;

template <typename U, int BLOCK, int UNROLL, bool NT, bool XCD>
__global__ __launch_bounds__(BLOCK) void swap_kernel(const int32_t* __restrict__ hdr, int runs_word,
                                                     const RunPair* __restrict__ runs,
                                                     const DirEntry* __restrict__ dir,
                                                     const unsigned char* __restrict__ in,
                                                     unsigned char* __restrict__ out, int32_t total,
                                                     int64_t row_bytes, int32_t tile_rows, int32_t n_tiles) {
  if (hdr[kHdrStatus] != THD_OK) return;  // a failed build writes nothing
  const int32_t n_runs = hdr[runs_word];
  const int32_t per_xcd = (n_tiles + kXcds - 1) / kXcds;
  const int32_t n_slots = XCD ? per_xcd * kXcds : n_tiles;
  for (int32_t slot = blockIdx.x; slot < n_slots; slot += gridDim.x) {
    const int32_t tile = XCD ? (slot % kXcds) * per_xcd + slot / kXcds : slot;
    if (tile >= n_tiles) continue;
    int32_t r0 = static_cast<int32_t>(static_cast<int64_t>(tile) * tile_rows);
    const int32_t r1 = static_cast<int32_t>(min(static_cast<int64_t>(total), static_cast<int64_t>(r0) + tile_rows));
    // First piece: one directory load covers the usual case where no run
    // starts between the directory row (a multiple of 16) and r0.
    const DirEntry e = dir[r0 >> kDirShift];
    int32_t k, in_row, run_end;
    if (r0 < e.run_end) {
      k = e.run;
      in_row = e.in + (r0 & (kDirBlock - 1));
      run_end = e.run_end;
    } else {
      k = e.run + 1;
      while (k + 1 < n_runs && runs[k + 1].out <= r0) ++k;
      if (k >= n_runs) continue;
      const RunPair run = runs[k];
      if (run.out > r0) continue;
      in_row = run.in + (r0 - run.out);
      run_end = (k + 1 < n_runs) ? runs[k + 1].out : total;
    }
    while (true) {
      const int32_t piece_end = min(r1, run_end);
      const U* src = reinterpret_cast<const U*>(in + static_cast<int64_t>(in_row) * row_bytes);
      U* dst = reinterpret_cast<U*>(out + static_cast<int64_t>(r0) * row_bytes);
      const int64_t n_units = static_cast<int64_t>(piece_end - r0) * row_bytes / static_cast<int64_t>(sizeof(U));
      copy_span<U, BLOCK, UNROLL, NT>(src, dst, n_units);
      r0 = piece_end;
      if (r0 >= r1 || ++k >= n_runs) break;
      const RunPair run = runs[k];
      if (run.out != r0) break;  // runs tile the output rows; never trust anything else
      in_row = run.in;
      run_end = (k + 1 < n_runs) ? runs[k + 1].out : total;
    }
  }
}

struct Shape {
  int32_t tile_rows, n_tiles, grid;
};

template <typename U, int BLOCK, int UNROLL>
hipError_t launch_typed(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir, const void* in,
                        void* out, int32_t total, int64_t row_bytes, const Shape& sh, bool nt, bool xcd,
                        hipStream_t stream) {
  const auto* i8 = static_cast<const unsigned char*>(in);
  auto* o8 = static_cast<unsigned char*>(out);
#define THD_LAUNCH(NT_, X_)                                                                                      \
  hipLaunchKernelGGL((swap_kernel<U, BLOCK, UNROLL, NT_, X_>), dim3(sh.grid), dim3(BLOCK), 0, stream, hdr,       \
                     runs_word, runs, dir, i8, o8, total, row_bytes, sh.tile_rows, sh.n_tiles)
  if (nt) {
    if (xcd) THD_LAUNCH(true, true);
    else THD_LAUNCH(true, false);
  } else {
    if (xcd) THD_LAUNCH(false, true);
    else THD_LAUNCH(false, false);
  }
#undef THD_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swap(const int32_t* hdr, const RunPair* runs, int runs_word, const DirEntry* dir, const void* in,
                       void* out, int32_t total, int64_t row_bytes, const SwapLaunch& cfg, hipStream_t stream) {
  // Widest unit that divides the row size and both base addresses.
  const uint64_t align_bits = static_cast<uint64_t>(row_bytes) | reinterpret_cast<uintptr_t>(in) |
                              reinterpret_cast<uintptr_t>(out);
  int unit = 16;
  while (unit > 1 && (align_bits & (unit - 1))) unit >>= 1;

  // Launch shape.  Measured on MI355X: the swap streams best when each
  // workgroup copies about one row -- 4 KiB tiles of 128 threads for rows
  // under 8 KiB; one row per workgroup in XCD-grouped order for rows of 8 KiB
  // and more, 512 threads up to 4 GiB per buffer and 256 beyond (an empirical
  // split: 256 wins by ~2 % on the 16 GiB 1M-token batch, 512 by ~1-2 % on
  // 1-2 GiB batches).  Every field can be overridden for sweeps.
  const bool big_rows = unit == 16 && row_bytes >= 8192;
  const bool huge = static_cast<int64_t>(total) * row_bytes >= (int64_t{4} << 30);
  const int64_t tile_bytes = cfg.tile_bytes > 0 ? cfg.tile_bytes : (big_rows ? row_bytes : (unit == 16 ? 4096 : 8192));
  int block = cfg.block_threads > 0 ? cfg.block_threads : (unit == 16 ? (big_rows ? (huge ? 256 : 512) : 128) : 256);
  const bool xcd = cfg.tile_order == 2 || (cfg.tile_order == 0 && big_rows);

  int64_t tile_rows = (tile_bytes + row_bytes - 1) / row_bytes;
  if (tile_rows < 1) tile_rows = 1;
  if (tile_rows > (1 << 30)) tile_rows = 1 << 30;
  Shape sh;
  sh.tile_rows = static_cast<int32_t>(tile_rows);
  sh.n_tiles = static_cast<int32_t>((total + tile_rows - 1) / tile_rows);
  const int64_t slots = xcd ? static_cast<int64_t>((sh.n_tiles + kXcds - 1) / kXcds) * kXcds : sh.n_tiles;
  sh.grid = static_cast<int32_t>(slots);
  if (cfg.max_workgroups > 0 && sh.grid > cfg.max_workgroups) sh.grid = cfg.max_workgroups;
  if (sh.grid <= 0) return hipSuccess;
  const bool nt = cfg.nontemporal != 0;
#define THD_SWAP_ARGS hdr, runs, runs_word, dir, in, out, total, row_bytes, sh, nt, xcd, stream
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

}  // namespace thdcp
