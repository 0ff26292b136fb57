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
// (a multiple of 16 rows, about `tile_bytes` bytes); the route's directory
// gives the run covering the tile's first row in one load.  A workgroup walks
// the (usually one or two) runs that overlap its tile and streams each piece
// as a flat byte copy: consecutive lanes touch consecutive 16-byte vectors, so
// every wave-wide load and store is a fully coalesced 1 KiB access.  Run data
// is uniform across the workgroup and is read through scalar loads.
//
// The work is HBM-bound (2 * rows * row_bytes bytes, no arithmetic), so the
// kernel is built for bytes in flight: each thread issues UNROLL independent
// vector loads before its stores.
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

template <typename U, int BLOCK, int UNROLL, bool NT>
__global__ __launch_bounds__(BLOCK) void swap_kernel(const int32_t* __restrict__ hdr, int runs_word,
                                                     const RunPair* __restrict__ runs,
                                                     const int32_t* __restrict__ dir,
                                                     const unsigned char* __restrict__ in,
                                                     unsigned char* __restrict__ out, int32_t total,
                                                     int64_t row_bytes, int32_t tile_rows, int32_t n_tiles) {
  if (hdr[kHdrStatus] != THD_OK) return;  // a failed build writes nothing
  const int32_t n_runs = hdr[runs_word];
  for (int32_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    int32_t r0 = static_cast<int32_t>(static_cast<int64_t>(tile) * tile_rows);
    const int32_t r1 = static_cast<int32_t>(min(static_cast<int64_t>(total), static_cast<int64_t>(r0) + tile_rows));
    int32_t k = min(max(dir[r0 >> kDirShift], 0), n_runs - 1);
    while (r0 < r1 && k < n_runs) {
      const RunPair run = runs[k];
      const int32_t run_end = (k + 1 < n_runs) ? runs[k + 1].out : total;
      if (run_end <= r0) {  // the directory names the run holding r0; walking on only guards the table bounds
        ++k;
        continue;
      }
      if (run.out > r0) break;
      const int32_t piece_end = min(r1, run_end);
      const int64_t src_row = static_cast<int64_t>(run.in) + (r0 - run.out);
      const U* src = reinterpret_cast<const U*>(in + src_row * row_bytes);
      U* dst = reinterpret_cast<U*>(out + static_cast<int64_t>(r0) * row_bytes);
      const int64_t n_units = static_cast<int64_t>(piece_end - r0) * row_bytes / static_cast<int64_t>(sizeof(U));
      copy_span<U, BLOCK, UNROLL, NT>(src, dst, n_units);
      r0 = piece_end;
      ++k;
    }
  }
}

constexpr int kSwapBlock = 256;

template <typename U, int UNROLL>
hipError_t launch_typed(const int32_t* hdr, const RunPair* runs, int runs_word, const int32_t* dir, const void* in,
                        void* out, int32_t total, int64_t row_bytes, int32_t tile_rows, int32_t n_tiles,
                        int32_t grid, bool nt, hipStream_t stream) {
  const auto* i8 = static_cast<const unsigned char*>(in);
  auto* o8 = static_cast<unsigned char*>(out);
  if (nt)
    hipLaunchKernelGGL((swap_kernel<U, kSwapBlock, UNROLL, true>), dim3(grid), dim3(kSwapBlock), 0, stream, hdr,
                       runs_word, runs, dir, i8, o8, total, row_bytes, tile_rows, n_tiles);
  else
    hipLaunchKernelGGL((swap_kernel<U, kSwapBlock, UNROLL, false>), dim3(grid), dim3(kSwapBlock), 0, stream, hdr,
                       runs_word, runs, dir, i8, o8, total, row_bytes, tile_rows, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swap(const int32_t* hdr, const RunPair* runs, int runs_word, const int32_t* dir, const void* in,
                       void* out, int32_t total, int64_t row_bytes, const SwapLaunch& cfg, hipStream_t stream) {
  // Widest unit that divides the row size and both base addresses.
  const uint64_t align_bits = static_cast<uint64_t>(row_bytes) | reinterpret_cast<uintptr_t>(in) |
                              reinterpret_cast<uintptr_t>(out);
  int unit = 16;
  while (unit > 1 && (align_bits & (unit - 1))) unit >>= 1;

  int64_t tile_rows = (cfg.tile_bytes + row_bytes - 1) / row_bytes;
  tile_rows = ((tile_rows + kDirBlock - 1) / kDirBlock) * kDirBlock;
  if (tile_rows > (1 << 30)) tile_rows = 1 << 30;
  const int64_t n_tiles64 = (total + tile_rows - 1) / tile_rows;
  const int32_t n_tiles = static_cast<int32_t>(n_tiles64);
  int32_t grid = n_tiles;
  if (cfg.max_workgroups > 0 && grid > cfg.max_workgroups) grid = cfg.max_workgroups;
  if (grid <= 0) return hipSuccess;
  const bool nt = cfg.nontemporal != 0;
  const int32_t tr = static_cast<int32_t>(tile_rows);
  switch (unit) {
    case 16: return launch_typed<u32x4, 8>(hdr, runs, runs_word, dir, in, out, total, row_bytes, tr, n_tiles, grid, nt, stream);
    case 8:  return launch_typed<u32x2, 8>(hdr, runs, runs_word, dir, in, out, total, row_bytes, tr, n_tiles, grid, nt, stream);
    case 4:  return launch_typed<uint32_t, 8>(hdr, runs, runs_word, dir, in, out, total, row_bytes, tr, n_tiles, grid, nt, stream);
    case 2:  return launch_typed<uint16_t, 8>(hdr, runs, runs_word, dir, in, out, total, row_bytes, tr, n_tiles, grid, nt, stream);
    default: return launch_typed<uint8_t, 8>(hdr, runs, runs_word, dir, in, out, total, row_bytes, tr, n_tiles, grid, nt, stream);
  }
}

}  // namespace thdcp
