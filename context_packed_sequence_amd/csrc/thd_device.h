// Device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace thdcp {

// Exclusive prefix sum over a workgroup of kThreads threads (a multiple of
// 64, at most 1024).  Every thread must call it.  Returns the thread's
// exclusive offset and stores the workgroup total in *total.  s_wave is LDS
// scratch of kThreads / 64 + 1 elements.
template <int kThreads, typename T>
__device__ T block_exclusive_scan(T v, T* s_wave, T* total) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const T w = lane < kWaves ? s_wave[lane] : T(0);
    T xs = w;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const T y = __shfl_up(xs, o, 64);
      if (lane >= o) xs += y;
    }
    if (lane < kWaves) s_wave[lane] = xs - w;
    if (lane == kWaves - 1) s_wave[kWaves] = xs;
  }
  __syncthreads();
  const T excl = s_wave[wave] + x - v;
  *total = s_wave[kWaves];
  __syncthreads();
  return excl;
}

// Exclusive prefix maximum over a workgroup, same contract as
// block_exclusive_scan: thread i gets the maximum of v over threads < i
// (`lowest` for thread 0) and *total the maximum over all threads.
template <int kThreads, typename T>
__device__ T block_exclusive_max(T v, T lowest, T* s_wave, T* total) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  T x = v;  // inclusive maximum inside the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o, 64);
    if (lane >= o) x = x > y ? x : y;
  }
  T ex = __shfl_up(x, 1, 64);  // exclusive maximum inside the wave
  if (lane == 0) ex = lowest;
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const T w = lane < kWaves ? s_wave[lane] : lowest;
    T xs = w;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const T y = __shfl_up(xs, o, 64);
      if (lane >= o) xs = xs > y ? xs : y;
    }
    T prev = __shfl_up(xs, 1, 64);
    if (lane == 0) prev = lowest;
    if (lane < kWaves) s_wave[lane] = prev;
    if (lane == kWaves - 1) s_wave[kWaves] = xs;
  }
  __syncthreads();
  const T before = s_wave[wave];
  const T excl = before > ex ? before : ex;
  *total = s_wave[kWaves];
  __syncthreads();
  return excl;
}

}  // namespace thdcp
