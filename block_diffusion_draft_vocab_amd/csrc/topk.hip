// Stage 1: per-position log-softmax + top-K over the vocabulary.
//
// [DDTree] "핵심 아이디어" (core idea): one drafter forward gives a distribution
// over the vocabulary for every masked block position; the tree is built from
// their log-probabilities.  This pass reads the logits once from HBM.
//
// Design (HBM-bound stream, two launches, every phase a few hundred cycles):
//   topk_partial  grid (chunks, rows), 256 threads.  The chunk (<= 8192
//                 floats) is streamed into registers with 16-byte loads;
//                 block max, then the sum of exp(x - max); then the chunk's
//                 exact top-K:
//                   each wave takes T_w = the kw-th largest of its 64 lane
//                   maxima (kw = ceil(K / busy waves)); T = min over the
//                   waves, so at least K keys are >= T and every top-K key
//                   is;
//                   the few keys >= T are gathered in LDS (wave-aggregated
//                   appends) and each finds its rank by counting greater
//                   candidates (LDS broadcast reads).
//   topk_merge    one workgroup per row: log-sum-exp of the chunk partials;
//                 T = K-th largest of the first ceil(K/C) keys of the C
//                 sorted chunk lists; a binary search per list counts its
//                 keys >= T; those are compacted and ranked by counting.
// Keys are 64-bit: order-preserving bits of x on top, ~id below, so a larger
// key is a larger x and, among equal x, a smaller id.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "../../include/ddt.h"
#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

constexpr int kWaves = kTopkThreads / kWave;  // 4
constexpr int kCandCap = 512;
constexpr int kMergeMaxLists = kTopkMergeMaxLists;  // 256: one thread per list
constexpr int kMergeMaxKeys = kTopkMergeMaxKeys;    // 16384: staged in LDS by the merge
constexpr int kTopkPlanMaxLists = 128;  // chunk lists the logit pass itself plans
constexpr float kLog2e = 1.4426950408889634f;

// x + 0 turns -0 into +0 (and leaves every other value alone): the two
// zeros are the same logit and tie, so the smaller id must win.
__device__ __forceinline__ uint64_t make_key(float x, int id) {
  return ((uint64_t)f32_order(x + 0.0f) << 32) | (uint64_t)(~(uint32_t)id);
}

// Rank of key v among cand[0..n) (number of greater keys), reading the
// candidates two at a time as 16-byte LDS broadcasts (cand 16-byte aligned).
__device__ __forceinline__ int rank_among(const uint64_t* cand, int n, uint64_t v) {
  const uint4* c2 = reinterpret_cast<const uint4*>(cand);
  int rank = 0;
#pragma unroll 4
  for (int u = 0; u < n / 2; ++u) {
    const uint4 q = c2[u];
    const uint64_t a = ((uint64_t)q.y << 32) | q.x, b = ((uint64_t)q.w << 32) | q.z;
    rank += (a > v) + (b > v);
  }
  if (n & 1) rank += cand[n - 1] > v;
  return rank;
}

// A lower bound on the k-th largest of the wave's values (one per lane, 0
// meaning none), or 0 when fewer than k lanes hold one: the largest t whose
// low 16 bits are zero with at least k lanes holding v >= t, built from the
// top bit down, one ballot per bit.  That is the k-th largest with its low
// 16 bits cleared (the lane count above a bound only grows as the bound
// falls), so at least k lanes still reach it; for order-mapped floats it
// sits within 2^-7 of the value, and half the rounds of the exact search
// are saved.
__device__ __forceinline__ uint32_t wave_kth_largest_hi16(uint32_t v, int k) {
  // (v opaque to the compiler: each round's compare then feeds its ballot
  // directly instead of being re-materialised through a select)
  __asm__ volatile("" : "+v"(v));
  uint32_t t = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t c = t | (1u << b);
    if (__popcll(__builtin_amdgcn_ballot_w64(v >= c)) >= k) t = c;
  }
  return t;
}

struct PartialSmem {
  float wmax[kWaves];
  float wsum[kWaves];
  uint32_t thr[kWaves];
  int cand_n;
  alignas(16) uint64_t cand[kCandCap + kWave];  // + a spare slot per lane
};

template <int PER>
__global__ __launch_bounds__(kTopkThreads) void topk_partial_kernel(
    const float* __restrict__ logits, int64_t ld, int vocab, int k, float inv_t, int chunk_len,
    int n_chunks, uint64_t* __restrict__ part_key, float2* __restrict__ part_ms) {
  __shared__ PartialSmem sm;
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

  // element i of this thread is index c0 + ((i/4) * 256 + tid) * 4 + i%4.
  // Every load is issued unconditionally (out-of-range ones from c0), so
  // all of them are in flight together; the values are masked afterwards.
  float x[PER];
  if (vec) {
    float4 v[PER / 4];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int b = c0 + (q * kTopkThreads + tid) * 4;
      v[q] = load_f4_stream(rp + (b + 3 < c1 ? b : c0));
    }
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int b = c0 + (q * kTopkThreads + tid) * 4;
      const bool full = b + 3 < c1;
      x[4 * q + 0] = full ? v[q].x * inv_t : -INFINITY;
      x[4 * q + 1] = full ? v[q].y * inv_t : -INFINITY;
      x[4 * q + 2] = full ? v[q].z * inv_t : -INFINITY;
      x[4 * q + 3] = full ? v[q].w * inv_t : -INFINITY;
      if (!full && b < c1) {  // the one group that straddles the chunk end
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = b + e < c1 ? rp[b + e] * inv_t : -INFINITY;
      }
    }
  } else {
    float y[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
      y[i] = rp[idx < c1 ? idx : c0];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
      x[i] = idx < c1 ? y[i] * inv_t : -INFINITY;
    }
  }
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) tm = fmaxf(tm, x[i]);
  const float wm = wave_max_f(tm);
  if (lane == 0) sm.wmax[wid] = wm;
  if (tid == 0) sm.cand_n = 0;
  __syncthreads();

  // block max, this thread's sum of exp(x - max)
  const float M = fmaxf(fmaxf(sm.wmax[0], sm.wmax[1]), fmaxf(sm.wmax[2], sm.wmax[3]));
  float s = 0.f;
  if (M != -INFINITY) {
    // four running sums, so the exponentials do not wait on one add chain
    const float mb = M * kLog2e;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PER; ++i) s4[i & 3] += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, -mb));
    s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  }
  const float ws = wave_sum_f(s);
  if (lane == 0) sm.wsum[wid] = ws;
  // Per-wave threshold.  With nw non-empty waves and kw = ceil(k / nw):
  // a wave with >= kw valid lanes takes T_w = its kw-th largest lane
  // maximum, rounded down to 16 significant bits (>= kw of its keys are
  // >= T_w); a wave with fewer valid lanes
  // takes T_w = 0 (all its keys); an empty wave does not vote.  Then
  // T = min T_w leaves at least k keys (or all of them) >= T.
  {
    const int len = c1 - c0;
    const int lanes = min(kTopkThreads, (len + 3) / 4);
    const int nw = (lanes + kWave - 1) / kWave;
    const int kw = div_small(k + nw - 1, nw);  // (1 <= nw <= 4: no integer division)
    const bool me_valid = tm != -INFINITY;
    // a valid lane's order-mapped maximum is above f32_order(-inf) > 0, so 0
    // marks the lanes without a key
    const uint32_t t = wave_kth_largest_hi16(me_valid ? f32_order(tm) : 0u, kw);
    const uint64_t any_valid = __ballot(me_valid);
    if (lane == 0) sm.thr[wid] = any_valid == 0 ? 0xFFFFFFFFu : t;
  }
  __syncthreads();

  uint32_t T = sm.thr[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) T = sm.thr[w] < T ? sm.thr[w] : T;
  if (tid == 0) {
    const float S = (sm.wsum[0] + sm.wsum[1]) + (sm.wsum[2] + sm.wsum[3]);
    part_ms[(int64_t)row * n_chunks + chunk] = make_float2(M, S);
  }
  // gather the keys >= T (T == 0 means every valid key, i.e. every finite
  // x).  Only lanes whose own maximum reaches T hold such keys: they count
  // them, a wave prefix sum of the counts and one LDS atomic per wave give
  // each lane its first slot, and the lanes write their keys in element
  // order.  Waves without such a lane skip both passes.
  {
    const float tf = T == 0u ? -3.402823466e38f : f32_unorder(T);
    const bool holder = tm >= tf;
    int mine = 0;
    if (holder) {
#pragma unroll
      for (int i = 0; i < PER; ++i) mine += x[i] >= tf ? 1 : 0;
    }
    const int incl = wave_inclusive_scan(mine);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    int base = 0;
    if (lane == 0 && total > 0) base = atomicAdd(&sm.cand_n, total);
    base = __builtin_amdgcn_readfirstlane(base);
    if (holder) {
      int pos = base + incl - mine;
      if constexpr (PER <= 20) {
        // every element written, without a branch per element (the keys
        // not taken, or past the cap, go to the lane's spare slot); with
        // 32 values per thread the extra LDS writes cost more than the
        // branches they save
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const bool take = x[i] >= tf;
          const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
          sm.cand[take && pos < kCandCap ? pos : kCandCap + lane] = make_key(x[i], idx);
          pos += take ? 1 : 0;
        }
      } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          if (x[i] >= tf) {
            const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
            if (pos < kCandCap) sm.cand[pos] = make_key(x[i], idx);
            ++pos;
          }
        }
      }
    }
  }
  __syncthreads();

  uint64_t* out = part_key + ((int64_t)row * n_chunks + chunk) * k;
  const int n = sm.cand_n;
  if (n <= kCandCap) {
    for (int t = tid; t < n; t += kTopkThreads) {
      const uint64_t v = sm.cand[t];
      const int rank = rank_among(sm.cand, n, v);
      if (rank < k) out[rank] = v;
    }
    for (int j = n + tid; j < k; j += kTopkThreads) out[j] = 0ull;
    return;
  }
  // exact fallback for massive ties: k rounds of a block-wide arg-max
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = c0 + ((i >> 2) * kTopkThreads + tid) * 4 + (i & 3);
    key[i] = idx < c1 ? make_key(x[i], idx) : 0ull;
  }
  uint64_t* red = sm.cand;  // reused: kTopkThreads <= kCandCap
  uint64_t prev = ~0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (key[i] < prev && key[i] > b) b = key[i];
    __syncthreads();
    red[tid] = b;
    __syncthreads();
    for (int w = kTopkThreads / 2; w > 0; w >>= 1) {
      if (tid < w && red[tid + w] > red[tid]) red[tid] = red[tid + w];
      __syncthreads();
    }
    prev = red[0];
    if (tid == 0) out[j] = prev;
  }
}

struct MergeSmem {
  alignas(16) uint64_t cand[kCandCap];
  int cnt[kMergeMaxLists + 1];
  uint64_t thr;
  float lse;
};

// One workgroup per row over the n_chunks sorted lists of k keys.
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(
    const uint64_t* __restrict__ part_key, const float2* __restrict__ part_ms, int n_chunks,
    int k, int32_t* __restrict__ ids, float* __restrict__ logp, float* __restrict__ lse_out) {
  extern __shared__ __attribute__((aligned(16))) uint64_t lk[];  // [n_chunks * k]
  __shared__ MergeSmem sm;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int n = n_chunks * k;
  const uint64_t* lists = part_key + (int64_t)row * n;
  {
    // 16-byte staging (k * 8 bytes per list; n even whenever k is)
    const int n2 = n / 2;
    const uint4* src = reinterpret_cast<const uint4*>(lists);
    uint4* dst = reinterpret_cast<uint4*>(lk);
    for (int i = tid; i < n2; i += kTopkThreads) dst[i] = src[i];
    if ((n & 1) && tid == 0) lk[n - 1] = lists[n - 1];
  }
  if (tid < kWave) {
    // log-sum-exp of the chunk partials (<= 256 pairs, four per lane)
    float2 pp[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c = tid + h * kWave;
      pp[h] = c < n_chunks ? part_ms[(int64_t)row * n_chunks + c] : make_float2(-INFINITY, 0.f);
    }
    const float M = wave_max_f(fmaxf(fmaxf(pp[0].x, pp[1].x), fmaxf(pp[2].x, pp[3].x)));
    float s = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (pp[h].x != -INFINITY) s += pp[h].y * __builtin_amdgcn_exp2f((pp[h].x - M) * kLog2e);
    }
    const float S = wave_sum_f(s);
    if (lane == 0) sm.lse = M + logf(S);
  }
  __syncthreads();

  // T = k-th largest of the first mm keys of every list (n_chunks * mm >= k
  // keys, all distinct; mm is raised while the candidates fit 64, which
  // tightens T), so at least k keys of the row are >= T.  Chunk
  // lists shorter than k end in 0 keys, which are never >= T.
  const int mm = max(div_small(k + n_chunks - 1, n_chunks), min(k, div_small(kWave, n_chunks)));
  const int ns = n_chunks * mm;  // <= max(k + n_chunks, 64) <= 256
  if (tid < ns) {
    const int li = div_small(tid, mm);
    sm.cand[tid] = lk[li * k + (tid - li * mm)];
  }
  __syncthreads();
  if (tid < ns) {
    const uint64_t v = sm.cand[tid];
    if (rank_among(sm.cand, ns, v) == k - 1) sm.thr = v;
  }
  __syncthreads();
  const uint64_t T = sm.thr;
  // keys >= T per list: the list is sorted descending, binary search
  if (tid < n_chunks) {
    const uint64_t* L = lk + tid * k;
    int lo = 0, hi = k;  // first index with L[i] < T
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L[mid] >= T) lo = mid + 1;
      else hi = mid;
    }
    sm.cnt[tid] = lo;
  }
  __syncthreads();
  if (tid < kWave) {
    // exclusive scan of the <= 256 counts, four consecutive per lane
    int a[4], t = 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      a[h] = 4 * tid + h < n_chunks ? sm.cnt[4 * tid + h] : 0;
      t += a[h];
    }
    const int inc = wave_inclusive_scan(t);
    int ex = inc - t;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (4 * tid + h < n_chunks) sm.cnt[4 * tid + h] = ex;
      ex += a[h];
    }
    if (tid == kWave - 1) sm.cnt[n_chunks] = inc;
  }
  __syncthreads();
  const int nc = sm.cnt[n_chunks];  // >= k, about k
  const float lse = sm.lse;
  if (nc <= kCandCap) {
    if (tid < n_chunks) {
      const int o = sm.cnt[tid];
      const int len = (tid + 1 < n_chunks ? sm.cnt[tid + 1] : nc) - o;
      for (int j = 0; j < len; ++j) sm.cand[o + j] = lk[tid * k + j];
    }
    __syncthreads();
    for (int t = tid; t < nc; t += kTopkThreads) {
      const uint64_t v = sm.cand[t];
      const int rank = rank_among(sm.cand, nc, v);
      if (rank < k) {
        ids[(int64_t)row * k + rank] = (int32_t)(~(uint32_t)v);
        logp[(int64_t)row * k + rank] = f32_unorder((uint32_t)(v >> 32)) - lse;
      }
    }
  } else if (tid < kWave) {
    // massive ties: k-step merge of the list heads (lane owns lists lane,
    // lane + 64, lane + 128 and lane + 192)
    int pos[4] = {0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
      int who = -1;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
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

// Wave-level LDS hand-off: the wave's LDS writes are visible to all of its
// lanes afterwards (no block barrier; other waves are not involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kWaveCandCap = 512;  // keys >= T a wave ranks in LDS

// The same merge with one wave per row and no block barrier, for rows whose
// n = n_chunks * k keys fit R per lane (n <= 64 R) and whose threshold
// candidates fit C per lane (n_chunks * ceil(k / n_chunks) <= 64 C).  Each
// lane holds R keys of the row in registers; the threshold T comes from the
// candidates by a ballot search on their value bits; a wave scan of the
// per-lane counts of keys >= T places those keys in LDS, and each is ranked
// by counting the greater ones.  C = 2 serves rows where one
// candidate per lane would leave no more candidates than k (T would be the
// smallest list head and let most keys through).
template <int R, int C>
__global__ __launch_bounds__(kTopkThreads) void topk_merge_wave_kernel(
    const uint64_t* __restrict__ part_key, const float2* __restrict__ part_ms, int n_rows,
    int n_chunks, int k, int32_t* __restrict__ ids, float* __restrict__ logp,
    float* __restrict__ lse_out) {
  __shared__ alignas(16) uint64_t take_all[kWaves][kWaveCandCap + kWave];  // + a spare slot per lane
  const int wid = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (int)(blockDim.x / kWave) + wid;
  if (row >= n_rows) return;
  const int n = n_chunks * k;
  const uint64_t* lists = part_key + (int64_t)row * n;
  // candidates: the first mm keys of every list, as many as fit C per
  // lane (a larger set gives a tighter T and fewer keys to rank), at least
  // ceil(k / n_chunks) so that at least k candidates exist
  const int mm = max(div_small(k + n_chunks - 1, n_chunks), min(k, div_small(C * kWave, n_chunks)));
  const int ns = n_chunks * mm;  // <= 64 C (host check)

  // all global loads first: keys, threshold candidates, chunk (max, sum)
  // key r of this lane is key kidx(r) of the row: pairs of keys at 16-byte
  // steps across the wave, so each load instruction reads 1 KB contiguous
  // (the order of the keys inside the wave does not matter below: ranks
  // come from comparisons only).  An odd n (16-byte alignment not
  // guaranteed) takes 8-byte loads in the same order.
  auto kidx = [&](int r) { return 2 * (lane + kWave * (r >> 1)) + (r & 1); };
  uint64_t key[R];
  if ((n & 1) == 0) {
    const uint4* l4 = reinterpret_cast<const uint4*>(lists);
#pragma unroll
    for (int r = 0; r < R; r += 2) {
      const int i = lane + kWave * (r >> 1);
      const uint4 q = l4[2 * i < n ? i : 0];
      key[r] = ((uint64_t)q.y << 32) | q.x;
      key[r + 1] = ((uint64_t)q.w << 32) | q.z;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) key[r] = lists[kidx(r) < n ? kidx(r) : 0];
  }
  uint64_t c[C];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const int ci = lane + q * kWave;
    const int li = div_small(ci, mm);  // (float quotient: ci < 128)
    c[q] = lists[ci < ns ? li * k + (ci - li * mm) : 0];
  }
  const float2* ms = part_ms + (int64_t)row * n_chunks;
  const float2 p0 = ms[lane < n_chunks ? lane : 0];
  const float2 p1 = ms[lane + kWave < n_chunks ? lane + kWave : 0];

  // log-sum-exp of the chunk partials
  float lse;
  {
    const float a = lane < n_chunks ? p0.x : -INFINITY;
    const float b = lane + kWave < n_chunks ? p1.x : -INFINITY;
    const float M = wave_max_f(fmaxf(a, b));
    float s = 0.f;
    if (M != -INFINITY) {
      if (a != -INFINITY) s += p0.y * __builtin_amdgcn_exp2f((a - M) * kLog2e);
      if (b != -INFINITY) s += p1.y * __builtin_amdgcn_exp2f((b - M) * kLog2e);
    }
    lse = M + logf(wave_sum_f(s));
  }

  // T = the k-th largest candidate's value part (its upper 32 bits, the
  // order-mapped float), found from the top bit down with one ballot per
  // candidate slot and bit: the largest t with at least k candidates whose
  // value part is >= t.  Keys >= (t, 0) include every candidate at or above
  // the k-th, so at least k keys; ties on the value add a few.  (0 -- take
  // every key -- when fewer than k candidates are real keys: zero padding
  // ends short lists.)
  uint32_t hv[C];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    hv[q] = lane + q * kWave < ns ? (uint32_t)(c[q] >> 32) : 0u;
    // (opaque to the compiler, so every round's compare feeds its ballot
    // directly instead of being re-materialised through a select)
    __asm__ volatile("" : "+v"(hv[q]));
  }
  uint32_t tv = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tv | (1u << b);
    int cnt_ge = 0;
#pragma unroll
    for (int q = 0; q < C; ++q) cnt_ge += __popcll(__builtin_amdgcn_ballot_w64(hv[q] >= cand));
    if (cnt_ge >= k) tv = cand;
  }
  const uint64_t T = (uint64_t)tv << 32;

  // this lane's keys >= T
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) cnt += (kidx(r) < n) && key[r] >= T;
  const int inc = wave_inclusive_scan(cnt);
  const int nc = __builtin_amdgcn_readlane(inc, kWave - 1);
  int32_t* oid = ids + (int64_t)row * k;
  float* olp = logp + (int64_t)row * k;
  if (nc <= kWaveCandCap) {
    uint64_t* tw = take_all[wid];
    // every key is written, without a branch per key: the ones not taken
    // go to the lane's spare slot
    int o = inc - cnt;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool take = (kidx(r) < n) && key[r] >= T;
      tw[take ? o : kWaveCandCap + lane] = key[r];
      o += take ? 1 : 0;
    }
    wave_lds_sync();
    for (int t = lane; t < nc; t += kWave) {
      const uint64_t v = tw[t];
      const int rank = rank_among(tw, nc, v);
      if (rank < k) {
        oid[rank] = (int32_t)(~(uint32_t)v);
        olp[rank] = f32_unorder((uint32_t)(v >> 32)) - lse;
      }
    }
  } else {
    // massive ties: k-step merge of the list heads (lane owns lists lane
    // and lane + 64), reading the lists from global memory
    int pos[2] = {0, 0};
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
      int who = -1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cc = lane + h * kWave;
        if (cc < n_chunks && pos[h] < k) {
          const uint64_t hv = lists[cc * k + pos[h]];
          if (hv > best) {
            best = hv;
            who = h;
          }
        }
      }
      uint64_t wb = best;
#pragma unroll
      for (int d = kWave / 2; d > 0; d >>= 1) {
        const uint64_t o2 = shfl_xor_u64(wb, d);
        wb = o2 > wb ? o2 : wb;
      }
      if (best == wb && wb != 0 && who >= 0) ++pos[who];
      if (lane == 0) {
        oid[j] = (int32_t)(~(uint32_t)wb);
        olp[j] = f32_unorder((uint32_t)(wb >> 32)) - lse;
      }
    }
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = lse;
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
  if (n_chunks > kTopkPlanMaxLists) n_chunks = kTopkPlanMaxLists;
  if (n_chunks > 8192 / k) n_chunks = 8192 / k;
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
  return n_rows <= 65535 && p.chunk_len <= kTopkMaxChunk && p.n_chunks <= kTopkPlanMaxLists &&
         p.n_chunks * k <= 8192;
}

namespace {
// Partials of the allocation-free entry point: one array per GPU, zero at
// load and never cleared (the partial kernel writes every entry the merge
// reads).  Host code must not pass this name to a kernel: on the host it is
// only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[DDT_TOPK_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t topk_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with device dev current: that device's copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_topk(const float* logits, int64_t ld, int n_rows, int vocab, int k,
                       float inv_t, int32_t* ids, float* logp, float* lse, void* ws,
                       hipStream_t stream) {
  const TopkPlan p = topk_plan(n_rows, vocab, k);
  uint64_t* part_key = static_cast<uint64_t*>(ws);
  float2* part_ms = reinterpret_cast<float2*>(
      static_cast<char*>(ws) + align256((size_t)n_rows * p.n_chunks * k * sizeof(uint64_t)));
  // 20 floats per thread when the chunk fits them (fewer loads and
  // registers for the short chunks of a few rows), else 32
  if (p.chunk_len <= kTopkThreads * 20)
    hipLaunchKernelGGL(topk_partial_kernel<20>, dim3(p.n_chunks, n_rows), dim3(kTopkThreads), 0,
                       stream, logits, ld, vocab, k, inv_t, p.chunk_len, p.n_chunks, part_key,
                       part_ms);
  else
    hipLaunchKernelGGL(topk_partial_kernel<kTopkPerThread>, dim3(p.n_chunks, n_rows),
                       dim3(kTopkThreads), 0, stream, logits, ld, vocab, k, inv_t, p.chunk_len,
                       p.n_chunks, part_key, part_ms);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(part_key, part_ms, n_rows, p.n_chunks, k, ids, logp, lse, stream);
}

hipError_t launch_topk_merge(const uint64_t* part_key, const float2* part_ms, int n_rows,
                             int n_chunks, int k, int32_t* ids, float* logp, float* lse,
                             hipStream_t stream) {
  const int n = n_chunks * k;
  const int ns_min = n_chunks * ((k + n_chunks - 1) / n_chunks);
  // candidates with one per lane; two per lane when that set would hold no
  // more than k keys
  const int ns1 = n_chunks * max((k + n_chunks - 1) / n_chunks, min(k, kWave / n_chunks));
  const int cand = ns1 <= k && ns_min <= 2 * kWave && n_chunks * min(k, 2 * kWave / n_chunks) > ns1
                       ? 2 : 1;
  if (n <= 64 * 32 && ns_min <= cand * kWave && n_chunks <= 2 * kWave) {
    // one wave per workgroup for a few rows (each row's merge on its own
    // CU), four for many
    const int wpb = n_rows <= 64 ? 1 : kWaves;
    const dim3 grid((n_rows + wpb - 1) / wpb);
#define DDT_MERGE_WAVE(RR, CC)                                                        \
  hipLaunchKernelGGL((topk_merge_wave_kernel<RR, CC>), grid, dim3(wpb * kWave), 0, stream, \
                     part_key, part_ms, n_rows, n_chunks, k, ids, logp, lse)
    if (cand == 1) {
      if (n <= 64 * 4) DDT_MERGE_WAVE(4, 1);
      else if (n <= 64 * 8) DDT_MERGE_WAVE(8, 1);
      else if (n <= 64 * 16) DDT_MERGE_WAVE(16, 1);
      else DDT_MERGE_WAVE(32, 1);
    } else {
      if (n <= 64 * 8) DDT_MERGE_WAVE(8, 2);
      else if (n <= 64 * 16) DDT_MERGE_WAVE(16, 2);
      else DDT_MERGE_WAVE(32, 2);
    }
#undef DDT_MERGE_WAVE
    return hipGetLastError();
  }
  const size_t smem = (size_t)n * sizeof(uint64_t);
  if (smem > 32 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(topk_merge_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n_rows), dim3(kTopkThreads), smem, stream, part_key,
                     part_ms, n_chunks, k, ids, logp, lse);
  return hipGetLastError();
}

}  // namespace ddt
