// Internal device helpers shared by the kernels of libddt (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddt {

constexpr int kWave = 64;  // CDNA wavefront width

// Order-preserving map float -> uint32: a < b  <=>  f32_order(a) < f32_order(b)
// (for non-NaN inputs, with -0 < +0).
__device__ __forceinline__ uint32_t f32_order(float x) {
  uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_unorder(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(b);
}

// Descending bitonic sort of n (a power of two) 64-bit keys held in LDS.
// Every thread of the block must call it; ends with a block barrier.
__device__ inline void bitonic_sort_desc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo | j;
        const uint64_t x = a[lo];
        const uint64_t y = a[hi];
        const bool desc = (lo & k) == 0;
        if (desc ? (x < y) : (x > y)) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Inclusive prefix sum across one wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(v, d, kWave);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive prefix sum of v over the block in thread order.  scratch needs
// blockDim.x/64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets
// the block sum.  Contains barriers: every thread must call it.
__device__ inline int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[nw] = run;
  }
  __syncthreads();
  const int res = scratch[wid] + inc - v;
  *total = scratch[nw];
  __syncthreads();
  return res;
}

// In-place exclusive scan of arr[0..n) (LDS) by the whole block; returns the
// total.  Each thread scans a contiguous run so the order is preserved.
__device__ inline int block_scan_array(int* arr, int n, int* scratch) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int b0 = min(n, (int)threadIdx.x * per);
  const int b1 = min(n, b0 + per);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += arr[i];
  int total;
  int run = block_exclusive_scan(s, scratch, &total);
  for (int i = b0; i < b1; ++i) {
    const int t = arr[i];
    arr[i] = run;
    run += t;
  }
  __syncthreads();
  return total;
}

}  // namespace ddt
