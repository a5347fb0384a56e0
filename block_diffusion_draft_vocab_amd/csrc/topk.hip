// Stage 1: per-position log-softmax + top-K over the vocabulary.
//
// [DDTree] "핵심 아이디어" (core idea): one drafter forward gives a distribution
// over the vocabulary for every masked block position; the tree is built from
// their log-probabilities.  This pass reads the logits once from HBM.
//
// Design (HBM-bound stream, two launches):
//   topk_partial  grid (chunks, rows).  Each workgroup streams one chunk of a
//                 row with 16-byte loads into registers, reduces (max, sum of
//                 exp) and extracts the chunk's exact top-K (block_topk).
//   topk_merge    one workgroup per row: log-sum-exp of the chunk partials and
//                 the top-K of the chunk lists (block_topk again).
// block_topk avoids sorting networks: a lower bound T on the K-th largest
// key is the K-th largest of 64..256 group maxima; the few keys >= T are
// gathered in LDS and ranked by counting.
// Keys are 64-bit: order-preserving bits of x on top, ~id below, so a larger
// key is a larger x and, among equal x, a smaller id.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

constexpr int kCandCap = 256;
constexpr int kMergeMaxLists = 2 * kWave;  // lists the merge wave can own
constexpr int kMergeMaxKeys = 8192;        // staged in LDS by the merge

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

struct SelectSmem {
  uint64_t tmax[kTopkThreads];
  uint64_t gmax[kTopkThreads];
  uint64_t cand[kCandCap];
  uint64_t thr;
  int cand_n;
};

// Top-k (k <= 128) of the 64-bit keys spread over the block, E per thread
// (0 = empty slot), written sorted descending to out[0..k).  Exact:
//   T = k-th largest of G group maxima (G = 64, 128 or 256 groups of
//       threads, the smallest with G >= 2k) -- at least k keys are >= T, so
//       every top-k key is >= T;
//   the keys >= T (about k of them) are gathered in LDS; each finds its
//   rank by counting the greater candidates and lands at out[rank].
// Keys are distinct (the low half is the token id), so ranks are too.
// More than kCandCap candidates (massive ties) fall back to k rounds of a
// block-wide arg-max.  Every thread must call it.
template <int E>
__device__ void block_topk(const uint64_t (&key)[E], int k, uint64_t* out, SelectSmem& sm) {
  const int tid = threadIdx.x;
  uint64_t tm = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) tm = key[e] > tm ? key[e] : tm;
  sm.tmax[tid] = tm;
  if (tid == 0) {
    sm.cand_n = 0;
    sm.thr = 1;
  }
  __syncthreads();
  const int G = k <= 32 ? 64 : (k <= 64 ? 128 : 256);
  uint64_t gm = 0;
  if (tid < G) {
    for (int t = tid; t < kTopkThreads; t += G) gm = sm.tmax[t] > gm ? sm.tmax[t] : gm;
    sm.gmax[tid] = gm;
  }
  __syncthreads();
  if (tid < G && gm != 0) {
    int rank = 0;
    for (int u = 0; u < G; ++u) rank += sm.gmax[u] > gm;
    if (rank == k - 1) sm.thr = gm;
  }
  __syncthreads();
  const uint64_t thr = sm.thr;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] >= thr) {
      const int pos = atomicAdd(&sm.cand_n, 1);
      if (pos < kCandCap) sm.cand[pos] = key[e];
    }
  }
  __syncthreads();
  const int n = sm.cand_n;
  if (n <= kCandCap) {
    if (tid < n) {
      const uint64_t v = sm.cand[tid];
      int rank = 0;
      for (int u = 0; u < n; ++u) rank += sm.cand[u] > v;
      if (rank < k) out[rank] = v;
    }
    for (int j = n + tid; j < k; j += kTopkThreads) out[j] = 0ull;
    return;
  }
  // exact fallback: k rounds of block-wide max below the previous pick
  uint64_t prev = ~0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t b = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] < prev && key[e] > b) b = key[e];
    __syncthreads();
    sm.tmax[tid] = b;
    __syncthreads();
    for (int w = kTopkThreads / 2; w > 0; w >>= 1) {
      if (tid < w && sm.tmax[tid + w] > sm.tmax[tid]) sm.tmax[tid] = sm.tmax[tid + w];
      __syncthreads();
    }
    prev = sm.tmax[0];
    if (tid == 0) out[j] = prev;
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_partial_kernel(
    const float* __restrict__ logits, int64_t ld, int vocab, int k, float inv_t, int chunk_len,
    int n_chunks, uint64_t* __restrict__ part_key, float2* __restrict__ part_ms) {
  __shared__ SelectSmem sm;
  __shared__ float red_m[kTopkThreads / kWave];
  __shared__ float red_s[kTopkThreads / kWave];

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
  uint64_t key[kTopkPerThread];
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) {
    const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
    const bool ok = idx < c1;
    if (ok) s += __expf(x[i] - m);
    key[i] = ok ? make_key(x[i], idx) : 0ull;
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
  block_topk<kTopkPerThread>(key, k, part_key + ((int64_t)row * n_chunks + chunk) * k, sm);
  if (tid == 0) {
    float M = red_m[0], S = red_s[0];
    for (int w = 1; w < kTopkThreads / kWave; ++w) ms_combine(M, S, red_m[w], red_s[w]);
    part_ms[(int64_t)row * n_chunks + chunk] = make_float2(M, S);
  }
}

// One workgroup per row.  The chunk lists (each sorted descending) are
// staged in LDS, then:
//   S = the first m entries of every list (m = ceil(2k / n_chunks), |S| <=
//       kCandCap), T = k-th largest of S -- k entries of S are >= T, so
//       every top-k entry of the row is >= T;
//   candidates = the prefix of every list that is >= T (about k entries);
//   each candidate's rank = number of greater candidates -> out[rank].
// Over kCandCap candidates (massive ties) falls back to a k-step merge of
// the list heads.  Also combines the chunks' (max, sum of exp) into the
// row's log-sum-exp.
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(
    const uint64_t* __restrict__ part_key, const float2* __restrict__ part_ms, int n_chunks,
    int k, int32_t* __restrict__ ids, float* __restrict__ logp, float* __restrict__ lse_out) {
  extern __shared__ uint64_t lk[];  // [n_chunks * k]
  __shared__ uint64_t cand[kCandCap];
  __shared__ int cnt[kMergeMaxLists + 1];
  __shared__ uint64_t thr_s;
  __shared__ float lse_s;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = n_chunks * k;
  const uint64_t* lists = part_key + (int64_t)row * n;
  for (int i = tid; i < n; i += kTopkThreads) lk[i] = lists[i];
  if (tid < kWave) {
    float m = -INFINITY, sm = 0.f;
    for (int c = tid; c < n_chunks; c += kWave) {
      const float2 p = part_ms[(int64_t)row * n_chunks + c];
      ms_combine(m, sm, p.x, p.y);
    }
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
      const float m2 = __shfl_xor(m, d, kWave);
      const float s2 = __shfl_xor(sm, d, kWave);
      ms_combine(m, sm, m2, s2);
    }
    if (tid == 0) {
      lse_s = m + logf(sm);
      thr_s = 1;
    }
  }
  __syncthreads();
  int mm = (2 * k + n_chunks - 1) / n_chunks;
  if (mm > k) mm = k;
  while (n_chunks * mm > kCandCap) --mm;
  const int ns = n_chunks * mm;
  if (tid < ns) {
    const uint64_t v = lk[(tid / mm) * k + (tid % mm)];
    if (v != 0) {
      int rank = 0;
      for (int u = 0; u < ns; ++u) rank += lk[(u / mm) * k + (u % mm)] > v;
      if (rank == k - 1) thr_s = v;
    }
  }
  __syncthreads();
  const uint64_t T = thr_s;
  if (tid < n_chunks) {
    int j = 0;
    while (j < k && lk[tid * k + j] >= T) ++j;
    cnt[tid] = j;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const int t = cnt[c];
      cnt[c] = run;
      run += t;
    }
    cnt[n_chunks] = run;
  }
  __syncthreads();
  const int nc = cnt[n_chunks];
  const float lse = lse_s;
  if (nc <= kCandCap) {
    if (tid < n_chunks) {
      const int o = cnt[tid];
      const int len = cnt[tid + 1] - o;
      for (int j = 0; j < len; ++j) cand[o + j] = lk[tid * k + j];
    }
    __syncthreads();
    if (tid < nc) {
      const uint64_t v = cand[tid];
      int rank = 0;
      for (int u = 0; u < nc; ++u) rank += cand[u] > v;
      if (rank < k) {
        ids[(int64_t)row * k + rank] = (int32_t)(~(uint32_t)v);
        logp[(int64_t)row * k + rank] = f32_unorder((uint32_t)(v >> 32)) - lse;
      }
    }
  } else if (tid < kWave) {
    // k-step merge of the list heads (lane owns lists lane and lane + 64)
    const int lane = tid;
    int pos[2] = {0, 0};
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
      int who = -1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + h * kWave;
        if (c < n_chunks && pos[h] < k) {
          const uint64_t hv = lk[c * k + pos[h]];
          if (hv > best) {
            best = hv;
            who = h;
          }
        }
      }
      uint64_t wb = best;
#pragma unroll
      for (int d = kWave / 2; d > 0; d >>= 1) {
        const uint64_t o = shfl_xor_u64(wb, d);
        wb = o > wb ? o : wb;
      }
      if (best == wb && wb != 0 && who >= 0) ++pos[who];
      if (lane == 0) {
        ids[(int64_t)row * k + j] = (int32_t)(~(uint32_t)wb);
        logp[(int64_t)row * k + j] = f32_unorder((uint32_t)(wb >> 32)) - lse;
      }
    }
  }
  if (lse_out != nullptr && tid == 0) lse_out[row] = lse;
}

}  // namespace

TopkPlan topk_plan(int n_rows, int vocab, int k) {
  // enough workgroups to cover the chip twice, chunks of at most 8192
  // floats, at most kMergeMaxLists chunk lists per row for the merge
  int n_chunks = (vocab + kTopkMaxChunk - 1) / kTopkMaxChunk;
  const int want = (512 + n_rows - 1) / n_rows;
  const int cap_small = vocab / 1024 > 1 ? vocab / 1024 : 1;
  int more = want < cap_small ? want : cap_small;
  if (more > n_chunks) n_chunks = more;
  if (n_chunks > kMergeMaxLists) n_chunks = kMergeMaxLists;
  if (n_chunks > kMergeMaxKeys / k) n_chunks = kMergeMaxKeys / k;
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
  return p.chunk_len <= kTopkMaxChunk && p.n_chunks <= kMergeMaxLists &&
         p.n_chunks * k <= kMergeMaxKeys;
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
  const size_t smem = (size_t)p.n_chunks * k * sizeof(uint64_t);
  if (smem > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_merge_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n_rows), dim3(kTopkThreads), smem, stream, part_key,
                     part_ms, p.n_chunks, k, ids, logp, lse);
  return hipGetLastError();
}

}  // namespace ddt
