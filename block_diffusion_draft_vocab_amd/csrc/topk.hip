// Stage 1: per-position log-softmax + top-K over the vocabulary.
//
// [DDTree] "핵심 아이디어" (core idea): one drafter forward gives a distribution
// over the vocabulary for every masked block position; the tree is built from
// their log-probabilities.  This pass reads the logits once from HBM.
//
// Design (HBM-bound stream, two launches):
//   topk_partial  grid (chunks, rows).  Each workgroup streams one chunk of a
//                 row with 16-byte loads into registers, reduces (max, sum of
//                 exp) and extracts the chunk's exact top-K:
//                   T = K-th largest of the per-thread maxima (a lower bound
//                       on the chunk's K-th largest value), candidates = all
//                       elements >= T (about K of them), bitonic sort in LDS.
//                 A rare overflow of the candidate buffer (massive ties) falls
//                 back to K rounds of block-wide arg-max, still exact.
//   topk_merge    one workgroup per row: log-sum-exp of the chunk partials,
//                 bitonic merge of the chunk top-K lists, log-probs out.
// Keys are 64-bit: order-preserving bits of x on top, ~id below, so a larger
// key is a larger x and, among equal x, a smaller id.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

constexpr int kCandCap = 512;
constexpr int kMergeMaxKeys = 16384;

__device__ __forceinline__ uint64_t make_key(float x, int id) {
  return ((uint64_t)f32_order(x) << 32) | (uint64_t)(~(uint32_t)id);
}

__device__ __forceinline__ void ms_combine(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    m = M;
    s = 0.f;
    return;
  }
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

__global__ __launch_bounds__(kTopkThreads) void topk_partial_kernel(
    const float* __restrict__ logits, int64_t ld, int vocab, int k, float inv_t, int chunk_len,
    int n_chunks, uint64_t* __restrict__ part_key, float2* __restrict__ part_ms) {
  __shared__ uint64_t tmax[kTopkThreads];
  __shared__ uint64_t cand[kCandCap];
  __shared__ float red_m[kTopkThreads / kWave];
  __shared__ float red_s[kTopkThreads / kWave];
  __shared__ int cand_n;

  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const float* rp = logits + (int64_t)row * ld;
  const int c0 = chunk * chunk_len;
  const int c1 = min(vocab, c0 + chunk_len);
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);

  float x[kTopkPerThread];
#pragma unroll
  for (int q = 0; q < kTopkPerThread / 4; ++q) {
    const int base = c0 + (q * kTopkThreads + tid) * 4;
    if (vec && base + 3 < c1) {
      const float4 v = *reinterpret_cast<const float4*>(rp + base);
      x[4 * q + 0] = v.x * inv_t;
      x[4 * q + 1] = v.y * inv_t;
      x[4 * q + 2] = v.z * inv_t;
      x[4 * q + 3] = v.w * inv_t;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = base + e;
        x[4 * q + e] = idx < c1 ? rp[idx] * inv_t : -INFINITY;
      }
    }
  }

  // (max, sum exp) of this thread, then of the block
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) m = fmaxf(m, x[i]);
  float s = 0.f;
  uint64_t best = 0;
  if (m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) {
      const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
      if (idx < c1) {
        s += expf(x[i] - m);
        const uint64_t key = make_key(x[i], idx);
        best = key > best ? key : best;
      }
    }
  }
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) {
    const float m2 = __shfl_xor(m, d, kWave);
    const float s2 = __shfl_xor(s, d, kWave);
    ms_combine(m, s, m2, s2);
  }
  if ((tid & (kWave - 1)) == 0) {
    red_m[tid / kWave] = m;
    red_s[tid / kWave] = s;
  }
  tmax[tid] = best;
  if (tid == 0) cand_n = 0;
  __syncthreads();
  if (tid == 0) {
    float M = red_m[0], S = red_s[0];
    for (int w = 1; w < kTopkThreads / kWave; ++w) ms_combine(M, S, red_m[w], red_s[w]);
    part_ms[(int64_t)row * n_chunks + chunk] = make_float2(M, S);
  }

  // threshold: K-th largest per-thread maximum
  bitonic_sort_desc(tmax, kTopkThreads);
  uint64_t thr = tmax[k - 1];
  if (thr == 0) thr = 1;  // fewer than K non-empty threads: keep every element

#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) {
    const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
    if (idx < c1) {
      const uint64_t key = make_key(x[i], idx);
      if (key >= thr) {
        const int pos = atomicAdd(&cand_n, 1);
        if (pos < kCandCap) cand[pos] = key;
      }
    }
  }
  __syncthreads();
  const int n = cand_n;
  uint64_t* out = part_key + ((int64_t)row * n_chunks + chunk) * k;
  if (n <= kCandCap) {
    int M = 2;
    while (M < n) M <<= 1;
    for (int i = n + tid; i < M; i += kTopkThreads) cand[i] = 0;
    __syncthreads();
    bitonic_sort_desc(cand, M);
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? cand[j] : 0;
    return;
  }
  // exact fallback: K rounds of block-wide max below the previous pick
  uint64_t prev = ~0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) {
      const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
      if (idx < c1) {
        const uint64_t key = make_key(x[i], idx);
        if (key < prev && key > b) b = key;
      }
    }
    __syncthreads();
    tmax[tid] = b;
    __syncthreads();
    for (int w = kTopkThreads / 2; w > 0; w >>= 1) {
      if (tid < w && tmax[tid + w] > tmax[tid]) tmax[tid] = tmax[tid + w];
      __syncthreads();
    }
    prev = tmax[0];
    if (tid == 0) out[j] = prev;
  }
}

__global__ __launch_bounds__(256) void topk_merge_kernel(
    const uint64_t* __restrict__ part_key, const float2* __restrict__ part_ms, int n_chunks,
    int k, int32_t* __restrict__ ids, float* __restrict__ logp, float* __restrict__ lse_out) {
  extern __shared__ uint64_t buf[];
  __shared__ float lse_s;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = n_chunks * k;
  int M = 2;
  while (M < n) M <<= 1;
  const uint64_t* src = part_key + (int64_t)row * n;
  for (int i = tid; i < M; i += blockDim.x) buf[i] = i < n ? src[i] : 0;
  if (tid == 0) {
    float m = -INFINITY, s = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
      const float2 p = part_ms[(int64_t)row * n_chunks + c];
      ms_combine(m, s, p.x, p.y);
    }
    lse_s = m + logf(s);
  }
  __syncthreads();
  bitonic_sort_desc(buf, M);
  const float lse = lse_s;
  for (int j = tid; j < k; j += blockDim.x) {
    const uint64_t key = buf[j];
    const float x = f32_unorder((uint32_t)(key >> 32));
    ids[(int64_t)row * k + j] = (int32_t)(~(uint32_t)key);
    logp[(int64_t)row * k + j] = x - lse;
  }
  if (lse_out != nullptr && tid == 0) lse_out[row] = lse;
}

}  // namespace

TopkPlan topk_plan(int n_rows, int vocab, int k) {
  // enough workgroups to cover the chip twice, chunks of at most 8192
  // floats, and at most kMergeMaxKeys keys for the per-row merge
  int n_chunks = (vocab + kTopkMaxChunk - 1) / kTopkMaxChunk;
  const int want = (512 + n_rows - 1) / n_rows;
  const int cap_small = vocab / 1024 > 1 ? vocab / 1024 : 1;
  int more = want < cap_small ? want : cap_small;
  if (more > n_chunks) n_chunks = more;
  const int cap_merge = kMergeMaxKeys / k;
  if (n_chunks > cap_merge) n_chunks = cap_merge;
  int chunk_len = (vocab + n_chunks - 1) / n_chunks;
  chunk_len = (chunk_len + 3) & ~3;
  n_chunks = (vocab + chunk_len - 1) / chunk_len;
  return {n_chunks, chunk_len};
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t topk_workspace_bytes(int n_rows, int vocab, int k) {
  const TopkPlan p = topk_plan(n_rows, vocab, k);
  return align256((size_t)n_rows * p.n_chunks * k * sizeof(uint64_t)) +
         align256((size_t)n_rows * p.n_chunks * sizeof(float2));
}

bool topk_supported(int n_rows, int vocab, int k) {
  const TopkPlan p = topk_plan(n_rows, vocab, k);
  return p.chunk_len <= kTopkMaxChunk && (int64_t)p.n_chunks * k <= kMergeMaxKeys;
}

hipError_t launch_topk(const float* logits, int64_t ld, int n_rows, int vocab, int k,
                       float inv_t, int32_t* ids, float* logp, float* lse, void* ws,
                       hipStream_t stream) {
  const TopkPlan p = topk_plan(n_rows, vocab, k);
  uint64_t* part_key = static_cast<uint64_t*>(ws);
  float2* part_ms = reinterpret_cast<float2*>(
      static_cast<char*>(ws) + align256((size_t)n_rows * p.n_chunks * k * sizeof(uint64_t)));
  hipLaunchKernelGGL(topk_partial_kernel, dim3(p.n_chunks, n_rows), dim3(kTopkThreads), 0,
                     stream, logits, ld, vocab, k, inv_t, p.chunk_len, p.n_chunks, part_key,
                     part_ms);
  int M = 2;
  while (M < p.n_chunks * k) M <<= 1;
  const size_t smem = (size_t)M * sizeof(uint64_t);
  if (smem > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_merge_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n_rows), dim3(256), smem, stream, part_key,
                     part_ms, p.n_chunks, k, ids, logp, lse);
  return hipGetLastError();
}

}  // namespace ddt
