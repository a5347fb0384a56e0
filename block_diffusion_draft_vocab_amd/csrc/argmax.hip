// Target argmax over the vocabulary: the verifier's greedy token per slot.
//
// [DDTree] "방법론 자세히 보기" (method in detail): the target runs once over
// the flattened tree and the verifier compares its outputs with the tree;
// under greedy decoding the target's output at a slot is its most probable
// next token, the arg-max of that slot's logits.  ddt_accept_compact walks
// the tree against these tokens.
//
// Design (one HBM stream, about three vector ops per float):
//   argmax_partial  grid (chunks, rows), 256 threads, PER floats per thread
//                   read with 16-byte non-temporal loads, all in flight
//                   together.
//                   Thread max, wave max (DPP); each lane finds the first of
//                   its elements equal to the wave max (a reverse select
//                   chain, no branches) and the wave takes the smallest such
//                   index; one barrier combines the four waves.  A chunk's
//                   result is one 64-bit key: order-preserving bits of the
//                   max on top, ~index below, so a larger key is a larger
//                   value and, among equal values, a smaller index.
//   argmax_merge    one wave per row: max of the row's chunk keys.  Not
//                   launched when a row is a single chunk (the partial then
//                   writes the id itself).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

constexpr int kAmWaves = kArgmaxThreads / kWave;  // 4

__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  return ((uint64_t)f32_order(v) << 32) | (uint64_t)(~idx);
}

template <int PER>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(
    const float* __restrict__ logits, int64_t ld, int vocab, int chunk_len, int n_chunks,
    uint64_t* __restrict__ part, int32_t* __restrict__ ids, float* __restrict__ maxv) {
  __shared__ uint64_t wkey[kAmWaves];
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const float* rp = logits + (int64_t)row * ld;
  const int c0 = chunk * chunk_len;
  const int c1 = min(vocab, c0 + chunk_len);
  // 16-byte loads need aligned rows and at least one whole 4-float group
  // (c0 is a multiple of 4, so the group at c0 is then in bounds)
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0) &&
                   c1 - c0 >= 4;

  // Element i of this thread is index c0 + ((i/4) * 256 + tid) * 4 + i%4.
  // Every load is issued unconditionally: a position past the chunk end
  // reads a copy of an element of the group at c0 instead.  Such copies
  // cannot change the max, and a copy that ties the max carries an index
  // >= c1, larger than that of its original (lane 0 of wave 0 holds c0),
  // so the smallest-index rule never picks it.  Within a thread all real
  // elements come before the copies.
  float x[PER];
  if (vec) {
    float4 v[PER / 4];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int b = c0 + (q * kArgmaxThreads + tid) * 4;
      v[q] = load_f4_stream(rp + (b + 3 < c1 ? b : c0));
    }
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      x[4 * q + 0] = v[q].x;
      x[4 * q + 1] = v[q].y;
      x[4 * q + 2] = v[q].z;
      x[4 * q + 3] = v[q].w;
      const int b = c0 + (q * kArgmaxThreads + tid) * 4;
      if (b + 3 >= c1 && b < c1) {  // the one group that straddles the chunk end
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = rp[b + e < c1 ? b + e : c0];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = c0 + ((i >> 2) * kArgmaxThreads + tid) * 4 + (i & 3);
      x[i] = rp[idx < c1 ? idx : c0];
    }
  }
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) tm = fmaxf(tm, x[i]);
  // + 0 turns a -0 maximum into +0, so waves and chunks whose maxima are
  // zeros of different sign compare equal and the index decides
  const float wm = wave_max_f(tm) + 0.0f;
  // first position (in index order) of this thread's elements equal to wm
  int f = PER;
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) f = x[i] == wm ? i : f;
  const uint32_t mine =
      f < PER ? (uint32_t)(c0 + ((f >> 2) * kArgmaxThreads + tid) * 4 + (f & 3)) : 0xFFFFFFFFu;
  const uint32_t widx = wave_min_u32(mine);
  if (lane == 0) wkey[wid] = argmax_key(wm, widx);
  __syncthreads();
  if (tid == 0) {
    uint64_t best = wkey[0];
#pragma unroll
    for (int w = 1; w < kAmWaves; ++w) best = wkey[w] > best ? wkey[w] : best;
    if (n_chunks == 1) {
      ids[row] = (int32_t)(~(uint32_t)best);
      if (maxv != nullptr) maxv[row] = f32_unorder((uint32_t)(best >> 32));
    } else {
      part[(int64_t)row * n_chunks + chunk] = best;
    }
  }
}

// One wave per row over the row's chunk keys.
__global__ __launch_bounds__(kArgmaxThreads) void argmax_merge_kernel(
    const uint64_t* __restrict__ part, int n_chunks, int n_rows, int32_t* __restrict__ ids,
    float* __restrict__ maxv) {
  const int row = blockIdx.x * kAmWaves + threadIdx.x / kWave;
  if (row >= n_rows) return;
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t* p = part + (int64_t)row * n_chunks;
  uint64_t best = 0;
  for (int c = lane; c < n_chunks; c += kWave) best = p[c] > best ? p[c] : best;
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) {
    const uint64_t o = shfl_xor_u64(best, d);
    best = o > best ? o : best;
  }
  if (lane == 0) {
    ids[row] = (int32_t)(~(uint32_t)best);
    if (maxv != nullptr) maxv[row] = f32_unorder((uint32_t)(best >> 32));
  }
}

}  // namespace

ArgmaxPlan argmax_plan(int n_rows, int vocab) {
  (void)n_rows;
  int n_chunks = (vocab + kArgmaxMaxChunk - 1) / kArgmaxMaxChunk;
  int chunk_len = (vocab + n_chunks - 1) / n_chunks;
  chunk_len = (chunk_len + 3) & ~3;
  n_chunks = (vocab + chunk_len - 1) / chunk_len;
  return {n_chunks, chunk_len};
}

size_t argmax_workspace_bytes(int n_rows, int vocab) {
  const ArgmaxPlan p = argmax_plan(n_rows, vocab);
  return p.n_chunks == 1 ? 0 : (size_t)n_rows * p.n_chunks * sizeof(uint64_t);
}

hipError_t launch_argmax(const float* logits, int64_t ld, int n_rows, int vocab, int32_t* ids,
                         float* maxv, void* ws, hipStream_t stream) {
  const ArgmaxPlan p = argmax_plan(n_rows, vocab);
  uint64_t* part = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(argmax_partial_kernel<kArgmaxPerThread>, dim3(p.n_chunks, n_rows),
                     dim3(kArgmaxThreads), 0, stream, logits, ld, vocab, p.chunk_len, p.n_chunks,
                     part, ids, maxv);
  if (p.n_chunks > 1)
    hipLaunchKernelGGL(argmax_merge_kernel, dim3((n_rows + kAmWaves - 1) / kAmWaves),
                       dim3(kArgmaxThreads), 0, stream, part, p.n_chunks, n_rows, ids, maxv);
  return hipGetLastError();
}

}  // namespace ddt
