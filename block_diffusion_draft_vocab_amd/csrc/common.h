// Internal device helpers shared by the kernels of libddt (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// x / d and x % d for x >= 0 and d > 0 the same across the wave: a shift
// and a mask when d is a power of two (the usual head-group sizes and
// top-K widths), else the division.
__device__ __forceinline__ int divmod_u(int x, int d, int& rem) {
  if ((d & (d - 1)) == 0) {
    rem = x & (d - 1);
    return x >> __builtin_ctz((unsigned)d);
  }
  const int q = (int)((unsigned)x / (unsigned)d);
  rem = x - q * d;
  return q;
}

// Division by a divisor d >= 1 fixed for a launch, of any n in [0, 2^31):
// with l = ceil(log2 d), m = ceil(2^(31+l) / d) fits 32 bits, and
// n m / 2^(31+l) exceeds n / d by n e / (d 2^(31+l)) with e = m d - 2^(31+l)
// < d <= 2^l, which stays below 1/d, so the floor is the quotient
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  The host computes (m, s); a uniform quotient is
// then a scalar multiply and shift, a per-lane one three vector operations,
// instead of the ~30-instruction reciprocal sequence of a runtime division.
struct FastDiv {
  uint32_t m;
  uint32_t s;
  uint32_t d;
};
inline FastDiv make_fastdiv(uint32_t d) {
  if (d == 0) d = 1;  // (unused divisors: any valid value)
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.s = 31 + l;
  f.m = (uint32_t)(((1ull << f.s) + d - 1) / d);
  f.d = d;
  return f;
}
__host__ __device__ __forceinline__ int fdiv(int n, const FastDiv& f) {
  return (int)(((uint64_t)(uint32_t)n * f.m) >> f.s);
}
__host__ __device__ __forceinline__ int fdivmod(int n, const FastDiv& f, int& rem) {
  const int q = fdiv(n, f);
  rem = n - q * (int)f.d;
  return q;
}

// floor(a / b) for 0 <= a < 2^21 and b >= 1 (b may differ across lanes):
// the float estimate from the reciprocal is within one of the quotient
// (relative error below 2^-22), and one correction step either way makes
// it exact.
__device__ __forceinline__ int div_small(int a, int b) {
  int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}

// 16-byte streaming load (non-temporal hint: the line is not kept for
// reuse), for data read exactly once such as a pass over the logits.
__device__ __forceinline__ float4 load_f4_stream(const float* p) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
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

// Inclusive prefix sum across one wavefront (DPP: shifts of 1, 2, 4, 8
// inside each row of 16 lanes, then the row totals broadcast forward).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
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

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Wave-wide max / sum, result in every lane: DPP within rows of 16, then the
// four row results.
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto dpp = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  v = max(v, dpp(v, std::integral_constant<int, 0xB1>{}));
  v = max(v, dpp(v, std::integral_constant<int, 0x4E>{}));
  v = max(v, dpp(v, std::integral_constant<int, 0x141>{}));
  v = max(v, dpp(v, std::integral_constant<int, 0x140>{}));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  auto dpp = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  v = min(v, dpp(v, std::integral_constant<int, 0xB1>{}));
  v = min(v, dpp(v, std::integral_constant<int, 0x4E>{}));
  v = min(v, dpp(v, std::integral_constant<int, 0x141>{}));
  v = min(v, dpp(v, std::integral_constant<int, 0x140>{}));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m, kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Descending bitonic sort of 64*R keys held by one wavefront, R per lane;
// element i lives in lane i/R, register i%R.  No LDS, no barriers.
template <int R>
__device__ inline void wave_sort_desc(uint64_t (&x)[R]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 2; k <= kWave * R; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = lane * R + r;
          const uint64_t y = shfl_xor_u64(x[r], j / R);
          const bool take_max = ((i & j) == 0) == ((i & k) == 0);
          x[r] = take_max ? (x[r] > y ? x[r] : y) : (x[r] < y ? x[r] : y);
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r & j) continue;
          const int i = lane * R + r;
          const uint64_t a = x[r], b = x[r | j];
          const bool desc = (i & k) == 0;
          const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
          x[r] = desc ? hi : lo;
          x[r | j] = desc ? lo : hi;
        }
      }
    }
  }
}

// One bitonic stage (k, j) on keys held R per lane, element index
// i = base + lane*R + r; j < 64*R, so partners live in the same wave.
template <int R>
__device__ __forceinline__ void bitonic_stage_in_wave(uint64_t (&x)[R], int base, int k, int j) {
  const int lane = threadIdx.x & (kWave - 1);
  if (j >= R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = base + lane * R + r;
      const uint64_t y = shfl_xor_u64(x[r], j / R);
      const bool take_max = ((i & j) == 0) == ((i & k) == 0);
      x[r] = take_max ? (x[r] > y ? x[r] : y) : (x[r] < y ? x[r] : y);
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r & j) continue;
      const int i = base + lane * R + r;
      const uint64_t a = x[r], b = x[r | j];
      const bool desc = (i & k) == 0;
      const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
      x[r] = desc ? hi : lo;
      x[r | j] = desc ? lo : hi;
    }
  }
}

// Descending bitonic sort of n keys in LDS (n a power of two, n = W*64*R
// for the first W waves of the block).  Keys stay in registers; only
// stages whose partner is in another wave go through LDS (two barriers
// each).  Every thread of the block calls it; ends with a barrier.
template <int R>
__device__ void block_sort_desc_r(uint64_t* a, int n) {
  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int span = kWave * R;
  const bool active = wid * span < n;
  const int base = wid * span;
  uint64_t x[R];
  if (active) {
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = a[base + lane * R + r];
  }
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= span) {
        __syncthreads();
        if (active) {
#pragma unroll
          for (int r = 0; r < R; ++r) a[base + lane * R + r] = x[r];
        }
        __syncthreads();
        if (active) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int i = base + lane * R + r;
            const uint64_t y = a[i ^ j];
            const bool take_max = ((i & j) == 0) == ((i & k) == 0);
            x[r] = take_max ? (x[r] > y ? x[r] : y) : (x[r] < y ? x[r] : y);
          }
        }
      } else if (active) {
        bitonic_stage_in_wave<R>(x, base, k, j);
      }
    }
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int r = 0; r < R; ++r) a[base + lane * R + r] = x[r];
  }
  __syncthreads();
}

// Dispatch: 4 keys per lane where possible (fewer waves, fewer cross-wave
// stages); sizes beyond 4 keys per lane of every wave use the LDS network.
__device__ inline void block_sort_desc(uint64_t* a, int n) {
  const int nw = blockDim.x / kWave;
  int waves = n / (kWave * 4);
  waves = waves < 1 ? 1 : (waves > nw ? nw : waves);
  const int R = n / (kWave * waves);
  switch (R) {
    case 1: block_sort_desc_r<1>(a, n); break;
    case 2: block_sort_desc_r<2>(a, n); break;
    case 4: block_sort_desc_r<4>(a, n); break;
    default: bitonic_sort_desc(a, n); break;
  }
}

}  // namespace ddt
