// Streaming ceilings of the chip: a read-only pass and a write-only pass over
// a buffer, in the tile shapes that stream fastest on MI355X.  The swap reads
// every byte of its input once and writes every byte of its output once, so
// no row permutation can run faster than a plain copy, and a copy can run no
// faster than the slower of its read and write streams.  These two kernels
// measure those streams on their own; they are not part of the transform.
//
// Shapes from sweeps on MI355X: 128-thread workgroups, 16-byte accesses, the
// tiles of each XCD in chunks of 256 consecutive tiles.  The read pass takes
// 4 KiB tiles (two non-temporal loads per thread), the write pass 2 KiB tiles
// (one store per thread) whose stores write through L2 to memory
// (StreamStore): 3-5 % faster than non-temporal stores on 0.5-8 GiB, the
// best of those sweeps (natural order was 2 % faster still up to 1 GiB and
// 9-10 % slower on 4-8 GiB).  Both issue their accesses from an unrolled
// loop of eight predicated slots per thread; on this chip that form streamed
// 5-10 % faster than a single access per thread.
#include <climits>

#include "thd_device.h"
#include "thd_internal.h"

namespace thdcp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamBlock = 128;
constexpr int kStreamSlots = 8;  // unrolled access slots per thread and loop pass
constexpr int kReadTileWords = 256;   // 4 KiB
constexpr int kWriteTileWords = 128;  // 2 KiB
constexpr int kStreamChunk = 256;
constexpr int kStreamXcds = 8;

__device__ inline int32_t stream_tile(int32_t slot, int32_t chunk) {
  const int32_t x = slot % kStreamXcds, j = slot / kStreamXcds;
  return chunk == 1 ? slot : ((j / chunk) * kStreamXcds + x) * chunk + j % chunk;
}

// Reads every word once and counts the words equal to `key`; a workgroup
// touches `count` only when one of its words matches, so the pass is a read
// stream whenever matches are rare.
__global__ __launch_bounds__(kStreamBlock) void read_stream_kernel(const u32x4* __restrict__ in, int64_t n_words,
                                                                   int32_t n_tiles, int32_t chunk, u32x4 key,
                                                                   uint32_t* __restrict__ count) {
  const int32_t tile = stream_tile(blockIdx.x, chunk);
  if (tile >= n_tiles) return;
  const int64_t u0 = static_cast<int64_t>(tile) * kReadTileWords;
  const int64_t u1 = min(n_words, u0 + kReadTileWords);
  uint32_t hits = 0;
  for (int64_t i = u0 + threadIdx.x; i < u1; i += kStreamBlock * kStreamSlots) {
    u32x4 v[kStreamSlots];
#pragma unroll
    for (int k = 0; k < kStreamSlots; ++k) {
      const int64_t w = i + static_cast<int64_t>(k) * kStreamBlock;
      v[k] = w < u1 ? __builtin_nontemporal_load(in + w) : ~key;
    }
#pragma unroll
    for (int k = 0; k < kStreamSlots; ++k)
      hits += (v[k].x == key.x && v[k].y == key.y && v[k].z == key.z && v[k].w == key.w) ? 1u : 0u;
  }
  if (hits) atomicAdd(count, hits);
}

// Writes word w as four copies of (uint32)w ^ seed; reads nothing.
__global__ __launch_bounds__(kStreamBlock) void write_stream_kernel(u32x4* __restrict__ out, int64_t n_words,
                                                                    int32_t n_tiles, int32_t chunk, uint32_t seed) {
  const int32_t tile = stream_tile(blockIdx.x, chunk);
  if (tile >= n_tiles) return;
  const int64_t u0 = static_cast<int64_t>(tile) * kWriteTileWords;
  const int64_t u1 = min(n_words, u0 + kWriteTileWords);
  const StreamStore st(out + u0, static_cast<int32_t>(u1 - u0) * 16);
  for (int64_t i = u0 + threadIdx.x; i < u1; i += kStreamBlock * kStreamSlots) {
#pragma unroll
    for (int k = 0; k < kStreamSlots; ++k) {
      const int64_t w = i + static_cast<int64_t>(k) * kStreamBlock;
      if (w < u1) {
        const uint32_t s = static_cast<uint32_t>(w) ^ seed;
        st(static_cast<int32_t>(w - u0), u32x4{s, s, s, s});
      }
    }
  }
}

// XCD-chunked grid over `tiles` tiles; false if it does not fit.
bool stream_grid(int64_t tiles, int32_t* chunk, int32_t* slots) {
  if (tiles > INT32_MAX / 2) return false;
  const int64_t per_xcd = (tiles + kStreamXcds - 1) / kStreamXcds;
  const int64_t c = kStreamChunk < per_xcd ? kStreamChunk : (per_xcd > 0 ? per_xcd : 1);
  const int64_t s = (tiles + kStreamXcds * c - 1) / (kStreamXcds * c) * kStreamXcds * c;
  if (s > INT32_MAX) return false;
  *chunk = static_cast<int32_t>(c);
  *slots = static_cast<int32_t>(s);
  return true;
}

}  // namespace

hipError_t launch_read_stream(const void* in, int64_t bytes, const uint32_t key[4], uint32_t* count,
                              hipStream_t stream) {
  const int64_t n_words = bytes / 16;
  const int64_t tiles = (n_words + kReadTileWords - 1) / kReadTileWords;
  if (tiles == 0) return hipSuccess;
  int32_t chunk = 1, slots = 0;
  if (!stream_grid(tiles, &chunk, &slots)) return hipErrorInvalidValue;
  const u32x4 k = {key[0], key[1], key[2], key[3]};
  hipLaunchKernelGGL(read_stream_kernel, dim3(static_cast<unsigned>(slots)), dim3(kStreamBlock), 0, stream,
                     static_cast<const u32x4*>(in), n_words, static_cast<int32_t>(tiles), chunk, k, count);
  return hipGetLastError();
}

hipError_t launch_write_stream(void* out, int64_t bytes, uint32_t seed, hipStream_t stream) {
  const int64_t n_words = bytes / 16;
  const int64_t tiles = (n_words + kWriteTileWords - 1) / kWriteTileWords;
  if (tiles == 0) return hipSuccess;
  int32_t chunk = 1, slots = 0;
  if (!stream_grid(tiles, &chunk, &slots)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(write_stream_kernel, dim3(static_cast<unsigned>(slots)), dim3(kStreamBlock), 0, stream,
                     static_cast<u32x4*>(out), n_words, static_cast<int32_t>(tiles), chunk, seed);
  return hipGetLastError();
}

}  // namespace thdcp
