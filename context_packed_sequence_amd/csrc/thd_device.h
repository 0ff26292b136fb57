// Device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace thdcp {

// Inclusive scan of one 64-lane wave with DPP lane moves instead of LDS
// permutes: four row_shr steps (1, 2, 4, 8) scan each row of 16 lanes, then
// row_bcast:15 carries each row's last lane into the next row (rows 1 and 3)
// and row_bcast:31 carries lane 31 into rows 2 and 3.  A lane whose source
// is outside its row, or whose row the step does not write, takes
// `identity`.  op must be associative with `identity` as its neutral value.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int32_t dpp_move(int32_t x, int32_t old) {
  return __builtin_amdgcn_update_dpp(old, x, kCtrl, kRowMask, 0xf, false);
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ int64_t dpp_move(int64_t x, int64_t old) {
  const int32_t lo = __builtin_amdgcn_update_dpp(static_cast<int32_t>(old), static_cast<int32_t>(x), kCtrl,
                                                 kRowMask, 0xf, false);
  const int32_t hi = __builtin_amdgcn_update_dpp(static_cast<int32_t>(old >> 32), static_cast<int32_t>(x >> 32),
                                                 kCtrl, kRowMask, 0xf, false);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_inclusive_scan(T x, T identity, Op op) {
  x = op(x, dpp_move<0x111, 0xf>(x, identity));  // row_shr:1
  x = op(x, dpp_move<0x112, 0xf>(x, identity));  // row_shr:2
  x = op(x, dpp_move<0x114, 0xf>(x, identity));  // row_shr:4
  x = op(x, dpp_move<0x118, 0xf>(x, identity));  // row_shr:8
  x = op(x, dpp_move<0x142, 0xa>(x, identity));  // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_move<0x143, 0xc>(x, identity));  // row_bcast:31 into rows 2 and 3
  return x;
}

struct ScanAdd {
  template <typename T>
  __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};
struct ScanMax {
  template <typename T>
  __device__ __forceinline__ T operator()(T a, T b) const { return a > b ? a : b; }
};

// Exclusive prefix sum over a workgroup of kThreads threads (a multiple of
// 64, at most 1024).  Every thread must call it.  Returns the thread's
// exclusive offset and stores the workgroup total in *total.  s_wave is LDS
// scratch of kThreads / 64 + 1 elements.
template <int kThreads, typename T>
__device__ T block_exclusive_scan(T v, T* s_wave, T* total) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const T x = wave_inclusive_scan(v, T(0), ScanAdd{});
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const T w = lane < kWaves ? s_wave[lane] : T(0);
    const T xs = wave_inclusive_scan(w, T(0), ScanAdd{});
    if (lane < kWaves) s_wave[lane] = xs - w;
    if (lane == kWaves - 1) s_wave[kWaves] = xs;
  }
  __syncthreads();
  const T excl = s_wave[wave] + x - v;
  *total = s_wave[kWaves];
  __syncthreads();
  return excl;
}

// Exclusive prefix sum over a workgroup with one barrier: each wave writes
// its total into half `parity` of s_wave, and after the barrier every wave
// reads all the totals and takes its own prefix from a wave scan of them
// (one DPP row holds up to 16 totals).  Consecutive calls must alternate
// `parity`: a call writes the half the previous call did not, and the half
// it reads is written again only two calls later, behind the next call's
// barrier, which no wave passes before every wave has read this call's
// totals (the barrier's release waits for the wave's LDS loads).  s_wave is
// LDS scratch of 2 * (kThreads / 64) elements, used by nothing else.
template <int kThreads>
__device__ __forceinline__ int32_t block_exclusive_scan_1b(int32_t v, int32_t* s_wave, int parity,
                                                           int32_t* total) {
  constexpr int kWaves = kThreads / 64;
  static_assert(kWaves <= 16, "the wave totals must fit one DPP row");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int32_t x = wave_inclusive_scan(v, 0, ScanAdd{});
  int32_t* buf = s_wave + parity * kWaves;
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  const int32_t w = lane < kWaves ? buf[lane] : 0;
  const int32_t xs = wave_inclusive_scan(w, 0, ScanAdd{});
  *total = __builtin_amdgcn_readlane(xs, kWaves - 1);
  const int32_t before = wave > 0 ? __builtin_amdgcn_readlane(xs, wave - 1) : 0;
  return before + x - v;
}

// K independent exclusive scans over a workgroup in one pass (one set of
// barriers): sums when kMax is false, maxima when it is true, with
// `identity` as the value before thread 0.  excl[k] is thread i's result,
// total[k] the workgroup's.  s is LDS scratch of K * (kThreads / 64 + 1).
template <int kThreads, int K, bool kMax>
__device__ void block_exclusive_multi(const int64_t (&v)[K], int64_t identity, int64_t* s, int64_t (&excl)[K],
                                      int64_t (&total)[K]) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t x[K], ex[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if constexpr (kMax) x[k] = wave_inclusive_scan(v[k], identity, ScanMax{});
    else x[k] = wave_inclusive_scan(v[k], identity, ScanAdd{});
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    ex[k] = dpp_move<0x138, 0xf>(x[k], identity);  // wave_shr:1, lane 0 takes identity
    if (lane == 63) s[k * (kWaves + 1) + wave] = x[k];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t w = lane < kWaves ? s[k * (kWaves + 1) + lane] : identity;
      int64_t xs;
      if constexpr (kMax) xs = wave_inclusive_scan(w, identity, ScanMax{});
      else xs = wave_inclusive_scan(w, identity, ScanAdd{});
      const int64_t prev = dpp_move<0x138, 0xf>(xs, identity);
      if (lane < kWaves) s[k * (kWaves + 1) + lane] = prev;
      if (lane == kWaves - 1) s[k * (kWaves + 1) + kWaves] = xs;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t before = s[k * (kWaves + 1) + wave];
    excl[k] = kMax ? (before > ex[k] ? before : ex[k]) : before + ex[k];
    total[k] = s[k * (kWaves + 1) + kWaves];
  }
  __syncthreads();
}

// Stores of streamed data that nothing in the launch reads back: raw buffer
// stores whose cache-policy operand carries the device-scope coherence bit
// (SC1) and the non-temporal hint (NT), so each store writes through its
// XCD's L2 towards memory instead of waiting there to be evicted.  Measured
// on MI355X (same box, interleaved, after a warm-up): a pure write stream of
// whole lines ran 3-5 % faster than with non-temporal stores (0.5-8 GiB),
// and a plain copy of whole lines 0.8-3 %, so both store this way.  A store that
// covers part of a 128-byte line reaches memory as a partial-line write, as
// the L2 no longer merges it with the line's other half: copies with
// misaligned outputs ran 10-16 % slower this way, and swaps of aligned rows
// gained under 1 %, so the swap kernels keep non-temporal stores.  The
// resource covers [base, base + bytes): the hardware drops a store outside
// it.  `base` must be uniform across the workgroup (the resource lives in
// scalar registers).
constexpr int kStreamStorePolicy = 16 | 2;  // policy operand bits: SC0 1, NT 2, SC1 16
constexpr int kBufferWord3 = 0x00020000;    // resource word 3: 32-bit data format, no index stride

typedef unsigned int StoreW4 __attribute__((ext_vector_type(4)));

struct StreamStore {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ StreamStore(void* base, int32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kBufferWord3)) {}
  // 16 bytes into word i, byte offset 16 * i
  __device__ __forceinline__ void operator()(int32_t i, StoreW4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, 16 * i, 0, kStreamStorePolicy);
  }
};

// Division of a non-negative int32 by a divisor that is fixed for a whole
// kernel: one multiply-high, an add and two shifts instead of the integer
// division sequence.  Round-up method of Granlund and Montgomery ("Division
// by Invariant Integers using Multiplication", 1994, Figure 4.1) with
// N = 32: l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, then
// floor(n / d) = (t + ((n - t) >> 1)) >> (l - 1) with t = mulhi(m, n).
// Valid for 0 <= n < 2^31 and 1 <= d < 2^31.
struct FastDiv {
  uint32_t m;
  int l;
  __host__ __device__ static FastDiv make(int32_t d) {
    FastDiv f{0, 0};
    while ((1u << f.l) < static_cast<uint32_t>(d)) ++f.l;
    const uint64_t num = (uint64_t{1} << 32) * ((uint64_t{1} << f.l) - static_cast<uint64_t>(d));
    f.m = static_cast<uint32_t>(num / static_cast<uint64_t>(d) + 1);
    return f;
  }
  __device__ __forceinline__ int32_t operator()(int32_t n) const {
    if (l == 0) return n;  // d == 1
    const uint32_t t = __umulhi(m, static_cast<uint32_t>(n));
    return static_cast<int32_t>((t + ((static_cast<uint32_t>(n) - t) >> 1)) >> (l - 1));
  }
};

}  // namespace thdcp
