// Stage 2: DDTree best-first top-B prefix tree, flattened, with parent/depth
// arrays and the ancestor bitmask.
//
// [DDTree] "방법론 자세히 보기" (method in detail): under the factorized draft
// distribution the optimal budget-B tree is the set of the B most probable
// prefixes; the page finds them with a best-first max-heap (B pops).  A heap
// pops one node at a time, which on a GPU means B dependent rounds.  This
// kernel computes the same set and the same pop order with a level-parallel
// selection that needs at most L rounds, one workgroup per request, all state
// in LDS:
//
//   G := the depth-1 candidates (already sorted), theta := B-th key of G
//   for depth d = 2..L:
//     parents := depth-(d-1) members of G, in G order (index j)
//     children (j, rank) with key > theta and (j+1)(rank+1) <= B; the
//       children of one parent form a descending run, whose length a binary
//       search over the ranks finds
//     G := top B of (G u runs), sorted: a bucket pass by score (atomic slot
//       per bucket, scan of the counts, scatter, rank within the bucket by
//       the full key) when the level has at most 8 candidates per thread,
//       pairwise merge-path rounds otherwise
//     theta := G[B-1]
//
// Why it is exact: a node's key is below its parent's and its elder
// sibling's, so the top-B set is closed under "parent" and "elder sibling";
// (j+1)(rank+1)-1 same-depth nodes precede child (j, rank); theta is the B-th
// key of a subset of all prefixes, hence never above the true B-th key.
// The canonical order (score desc, depth asc, parent slot asc, rank asc)
// uses the parent's slot only to break ties between equal-score nodes of one
// depth; among the nodes of one depth the parents' slot order equals their
// order inside G, so the level-local parent index j is used in its place.
//
// 64-bit key: [63:32] order-preserving score bits, [31:26] 63-depth,
// [17:0] 0x3FFFF - (j<<7 | rank); a larger key is earlier in the tree.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

__device__ __forceinline__ uint64_t tkey(float score, int depth, int pl, int rank) {
  const uint32_t low =
      ((uint32_t)(63 - depth) << 26) | (uint32_t)(0x3FFFF - ((pl << 7) | rank));
  return ((uint64_t)f32_order(score) << 32) | low;
}
__device__ __forceinline__ int key_depth(uint64_t key) {
  return 63 - (int)((uint32_t)key >> 26);
}
__device__ __forceinline__ int key_pr(uint64_t key) {
  return 0x3FFFF - (int)((uint32_t)key & 0x3FFFFu);
}
__device__ __forceinline__ float key_score(uint64_t key) {
  return f32_unorder((uint32_t)(key >> 32));
}

struct TreeLayout {
  int cand_cap;   // G plus every candidate a level can produce
  size_t bytes;
};

}  // namespace

static int nc_bound(int B, int k_tree) {
  long s = 0;
  for (int j = 0; j < B; ++j) {
    const int c = B / (j + 1);
    s += c < k_tree ? c : k_tree;
  }
  return (int)s;
}

static TreeLayout tree_layout(int L, int k_tree, int B) {
  const int Bp = B > 0 ? B : 1;
  const int cap = Bp + nc_bound(B, k_tree);
  size_t bytes = (size_t)cap * 8 * 2        // keys + merge buffer
                 + (size_t)L * k_tree * 4   // log-prob table
                 + (size_t)Bp * 4 * 3       // parent scores, counts, slots
                 + (size_t)(Bp + 2) * 4 * 3 // run offsets x2, parent slots
                 + 64 * 34 * 4 + 34 * 4 * 2 + 32 * 4;
  return {cap, bytes};
}

size_t tree_smem_bytes(int L, int k_tree, int budget) {
  return tree_layout(L, k_tree, budget).bytes;
}

namespace {

// Elements one thread carries through the register merge (levels with at
// most one candidate per thread, or more than this many, take the
// merge-path rounds).
constexpr int kMaxCarry = 8;
constexpr int kBuckets = 2048;  // buckets of the per-level sort (<= 64 x 34 - 1)

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

__global__ __launch_bounds__(1024) void tree_kernel(
    const float* __restrict__ logp, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ root_token, int L, int K, int k_tree, int B, int cand_cap,
    int32_t* __restrict__ n_nodes_out, int32_t* __restrict__ tok_out,
    int32_t* __restrict__ par_out, int32_t* __restrict__ dep_out,
    float* __restrict__ score_out, uint64_t* __restrict__ mask_out) {
  extern __shared__ uint64_t smem_u64[];
  const int Bp = B > 0 ? B : 1;
  uint64_t* keys = smem_u64;                       // [cand_cap]
  uint64_t* kbuf = keys + cand_cap;                // [cand_cap] merge ping-pong
  float* y = reinterpret_cast<float*>(kbuf + cand_cap);  // [L * k_tree]
  float* pscore = y + L * k_tree;                  // [Bp]
  int* rcnt = reinterpret_cast<int*>(pscore + Bp); // [Bp]
  int* slot_tab = rcnt + Bp;                       // [Bp]
  int* roff = slot_tab + Bp;                       // [Bp + 2] run offsets
  int* roff2 = roff + Bp + 2;                      // [Bp + 2]
  int* par_slot = roff2 + Bp + 2;                  // [Bp + 2]
  int* wcnt = par_slot + Bp + 2;                   // [64 chunks][34 depths]
  int* dcount = wcnt + 64 * 34;                    // [34]
  int* doff = dcount + 34;                         // [34]
  int* misc = doff + 34;                           // [32]

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int nt_log = __builtin_ctz((unsigned)nt);  // the launch gives 256, 512 or 1024 threads
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int n_max = B + 1;
  const int W = (n_max + 63) / 64;

  for (int i = tid; i < L * k_tree; i += nt) {
    int rk;
    const int d = divmod_u(i, k_tree, rk);
    y[i] = logp[((int64_t)r * L + d) * K + rk];
  }
  // gb: G (sorted, g keys) with the level's children appended after it;
  // obuf: the other buffer of the merge ping-pong
  uint64_t* gb = keys;
  uint64_t* obuf = kbuf;
  int g = min(k_tree, B);
  // a depth-1 score is the root's (0) plus the log-prob: -0 becomes +0
  // (read from the input, so G and the table fill in the same pass)
  for (int i = tid; i < g; i += nt) gb[i] = tkey(0.0f + logp[(int64_t)r * L * K + i], 1, 0, i);
  __syncthreads();
  uint64_t theta = (g == B && B > 0) ? gb[B - 1] : 0ull;
  const int nwaves = nt / kWave;
  // score of the best depth-(d-1) node: the rank-0 child of the previous
  // level's first parent (depth 1: rank 0 of row 0)
  float best_prev = 0.0f + y[0];

  int dmax = 1;  // deepest level that added nodes
  for (int d = 2; d <= L && g > 0; ++d) {
    // The level's best possible child is the rank-0 child of its first
    // parent (the best depth-(d-1) node, which is in G: it beat theta when
    // it was made, so the top-B cut kept it); every other child has a lower
    // or equal score and a later tie-break.  When that one does not beat
    // theta the level adds nothing, and neither does any deeper one.
    const float* yd = y + (d - 1) * k_tree;
    const float best_child = best_prev + yd[0];
    if (g == B && !(tkey(best_child, d, 0, 0) > theta)) break;
    best_prev = best_child;
    // parents: the depth d-1 members of G, numbered in G order.  At depth
    // 2 that is all of G (only depth-1 nodes so far), parent j = G[j], whose
    // score is 0 + y[j]; it is written with the run lengths below.
    // Deeper: a ballot per 64-position chunk, then the chunk counts summed
    // directly.
    int n = g;
    if (d > 2) {
      const int nchunk = (g + kWave - 1) / kWave;
      for (int c = wid; c < nchunk; c += nwaves) {
        const int q = c * kWave + lane;
        const bool is = q < g && key_depth(gb[q]) == d - 1;
        const uint64_t bal = __ballot(is);
        if (lane == 0) wcnt[c] = __popcll(bal);
        if (is) slot_tab[q] = __popcll(bal & lanemask_lt());
      }
      __syncthreads();
      // inclusive prefix of the chunk counts across the lanes of every wave
      // (nchunk <= 32); q / 64 is uniform across a wave in the loop below
      const int cinc = wave_inclusive_scan(lane < nchunk ? wcnt[lane] : 0);
      n = __builtin_amdgcn_readlane(cinc, kWave - 1);
      if (n == 0) break;
      for (int q = tid; q < g; q += nt) {
        const int c = q / kWave;
        const int pre = c > 0 ? __builtin_amdgcn_readlane(cinc, c - 1) : 0;
        const uint64_t kq = gb[q];
        if (key_depth(kq) == d - 1) pscore[pre + slot_tab[q]] = key_score(kq);
      }
      __syncthreads();
    }
    int nc;
    if (theta == 0ull && n <= kWave) {
      // No bound from G yet (fewer than B keys so far): every child with
      // (j+1)(c+1) <= B is a candidate, so parent j's run holds
      // min(k_tree, B / (j + 1)) children and the run offsets are one wave
      // scan, done by every wave alike: no search, no barrier.  The shuffles
      // run with every lane active (a uniform trip count).
      const int lenj = lane < n ? min(k_tree, div_small(B, lane + 1)) : 0;
      const int incj = wave_inclusive_scan(lenj);
      nc = __builtin_amdgcn_readlane(incj, kWave - 1);
      if (nc == 0) break;
      const float psj = lane < n ? (d == 2 ? 0.0f + y[lane] : pscore[lane]) : 0.f;
      const int exj = incj - lenj;
      const int items = n * k_tree;
      for (int base = 0; base < items; base += nt) {
        const int it = base + tid;
        int c;
        int j = divmod_u(it, k_tree, c);
        if (it >= items) j = c = 0;
        const int len = __shfl(lenj, j, kWave);
        const int o = __shfl(exj, j, kWave);
        const float ps = __shfl(psj, j, kWave);
        if (it < items && c < len) gb[g + o + c] = tkey(ps + yd[c], d, j, c);
      }
      // run starts: G at 0, parent j's run at g + its prefix, and the end
      if (lane < n) roff[1 + lane] = g + exj;
      if (lane == 0) {
        roff[0] = 0;
        roff[n + 1] = g + nc;
      }
      for (int b = tid; b <= kBuckets; b += nt) wcnt[b] = 0;  // bucket counts of the sort below
    } else {
      // run length of parent j: children (j, c) with key above theta and
      // (j+1)(c+1) <= B; keys fall with c, so a binary search finds it.
      // Thread t owns parents [t*per, t*per + per).
      // (n <= B < 2 * nt: the launch gives max(cand_cap, 1024) threads or more)
      const int per = (n + nt - 1) >> nt_log;
      int lens[2] = {0, 0};
      int mine = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = tid * per + u;
        int len = 0;
        if (u < per && j < n) {
          int lo = 0, hi = min(k_tree, div_small(B, j + 1));
          float ps;
          if (d == 2) {
            ps = 0.0f + y[j];  // the key of G[j], exactly
            pscore[j] = ps;    // read by the children pass, after a barrier
          } else {
            ps = pscore[j];
          }
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (tkey(ps + yd[mid], d, j, mid) > theta) lo = mid + 1;
            else hi = mid;
          }
          len = lo;
        }
        lens[u] = len;
        mine += len;
      }
      // block exclusive scan of the per-thread totals
      const int inc = wave_inclusive_scan(mine);
      if (lane == kWave - 1) misc[8 + wid] = inc;
      __syncthreads();
      const int winc = wave_inclusive_scan(lane < nwaves ? misc[8 + lane] : 0);
      const int wpre = wid > 0 ? __builtin_amdgcn_readlane(winc, wid - 1) : 0;
      nc = __builtin_amdgcn_readlane(winc, kWave - 1);
      {
        int o = wpre + inc - mine;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = tid * per + u;
          if (u < per && j < n) rcnt[j] = o;
          o += lens[u];
        }
      }
      if (nc == 0) break;
      __syncthreads();
      // children keys after G: run 0 = G at [0, g), run j+1 = parent j's
      const int items = n * k_tree;
      for (int it = tid; it < items; it += nt) {
        int c;
        const int j = divmod_u(it, k_tree, c);
        const int o = rcnt[j];
        const int len = (j + 1 < n ? rcnt[j + 1] : nc) - o;
        if (c < len) gb[g + o + c] = tkey(pscore[j] + yd[c], d, j, c);
      }
      for (int j = tid; j <= n + 1; j += nt)  // offsets of runs 0..n, and the end
        roff[j] = j == 0 ? 0 : (j <= n ? g + rcnt[j - 1] : g + nc);
      for (int b = tid; b <= kBuckets; b += nt) wcnt[b] = 0;  // bucket counts of the sort below
    }
    __syncthreads();
    const int total = g + nc;
    if (total <= kMaxCarry * nt) {
      // Top B of G and the runs by one bucket pass instead of merge rounds:
      // element e of [0, total) stays with thread e % nt (slot e / nt).
      // Its bucket falls with its score (linear in the score between the
      // level's extremes, so equal scores share a bucket); an atomic count
      // gives it a slot in its bucket; after a scan of the counts the keys
      // are scattered by (bucket start + slot), and each element's place is
      // its bucket's start plus the keys of its bucket above its own (keys
      // are distinct: depth, parent and rank are part of them).  Places
      // from B on are dropped.  Four barriers after the children's, where
      // pairwise merging takes one per round and a binary search per
      // element each round.
      int* bstart = wcnt;  // kBuckets + 1 counts, zeroed with the children
      // the extremes: the first and last key of every run (each wave alike)
      float smax = -INFINITY, smin = INFINITY;
      for (int i = lane; i <= n; i += kWave) {
        if (roff[i + 1] > roff[i]) {
          smax = fmaxf(smax, key_score(gb[roff[i]]));
          smin = fminf(smin, key_score(gb[roff[i + 1] - 1]));
        }
      }
      smax = wave_max_f(smax);
      smin = -wave_max_f(-smin);
      const float bscale = smax > smin ? (float)(kBuckets - 1) / (smax - smin) : 0.f;
      const int M = (total + nt - 1) >> nt_log;  // slots in use (uniform)
      uint64_t xk[kMaxCarry];
      int xb[kMaxCarry], xs[kMaxCarry];
#pragma unroll
      for (int m = 0; m < kMaxCarry; ++m) {
        xb[m] = -1;
        xs[m] = 0;
        xk[m] = 0ull;
        if (m >= M) continue;
        const int e = tid + m * nt;
        if (e < total) {
          xk[m] = gb[e];
          // bucket 0 holds the highest scores
          int bk = (int)((smax - key_score(xk[m])) * bscale);
          bk = bk < 0 ? 0 : (bk > kBuckets - 1 ? kBuckets - 1 : bk);
          xb[m] = bk;
          xs[m] = atomicAdd(&bstart[bk], 1);
        }
      }
      __syncthreads();
      // exclusive scan of the counts: wave w turns its segment of kBuckets /
      // nwaves buckets (rows of 64, read coalesced) into prefixes within the
      // segment and leaves the segment's total; a bucket's start is that
      // prefix plus the totals of the segments before it
      const int seg = kBuckets >> (nt_log - 6);  // kBuckets / nwaves (nwaves <= 16)
      {
        int run = 0;
        for (int r0 = 0; r0 < seg; r0 += kWave) {
          const int b = wid * seg + r0 + lane;
          const int c = bstart[b];
          const int inc = wave_inclusive_scan(c);
          bstart[b] = run + inc - c;
          run += __builtin_amdgcn_readlane(inc, kWave - 1);
        }
        if (lane == 0) misc[8 + wid] = run;
      }
      __syncthreads();
      // every element's bucket range [start, end), with all lanes active
      // (the shuffle reads lanes that the branches below would mask off):
      // the segment's prefix plus the totals of the segments before it
      const int tot_lane = lane < nwaves ? misc[8 + lane] : 0;
      const int seg_before = wave_inclusive_scan(tot_lane) - tot_lane;  // lane nwaves: total
      int xs0[kMaxCarry], xs1[kMaxCarry];
#pragma unroll
      for (int m = 0; m < kMaxCarry; ++m) {
        xs0[m] = xs1[m] = 0;
        if (m >= M) continue;
        const int b = xb[m] < 0 ? 0 : xb[m];
        xs0[m] = bstart[b] + __shfl(seg_before, b / seg, kWave);
        xs1[m] = (b + 1 < kBuckets ? bstart[b + 1] : 0) + __shfl(seg_before, (b + 1) / seg, kWave);
      }
#pragma unroll
      for (int m = 0; m < kMaxCarry; ++m)
        if (m < M && xb[m] >= 0) obuf[xs0[m] + xs[m]] = xk[m];
      __syncthreads();
#pragma unroll
      for (int m = 0; m < kMaxCarry; ++m) {
        if (m >= M || xb[m] < 0) continue;
        const int s0 = xs0[m], s1 = xs1[m];
        int above = 0;
        for (int j = s0; j < s1; ++j) above += obuf[j] > xk[m] ? 1 : 0;
        const int pos = s0 + above;
        if (pos < B) gb[pos] = xk[m];
      }
      __syncthreads();
    } else {
      // pairwise merge-path rounds: runs (2i, 2i+1) -> run i, every output
      // element placed independently by a binary search on its diagonal
      int R = n + 1;
      uint64_t* src = gb;
      uint64_t* dst = obuf;
      int* ro = roff;
      int* ro_next = roff2;
      while (R > 1) {
        const int Rn = (R + 1) >> 1;
        for (int p = tid; p < total; p += nt) {
          // pair i with ro[2i] <= p < ro[2i+2]
          int lo = 0, hi = Rn - 1;
          while (lo < hi) {
            const int m = (lo + hi + 1) >> 1;
            if (ro[2 * m] <= p) lo = m; else hi = m - 1;
          }
          const int a0 = ro[2 * lo];
          const int a1 = ro[2 * lo + 1];
          const int b1 = 2 * lo + 2 <= R ? ro[2 * lo + 2] : a1;
          const int la = a1 - a0, lb = b1 - a1;
          const int kk = p - a0;
          int l2 = kk - lb > 0 ? kk - lb : 0;
          int h2 = kk < la ? kk : la;
          while (l2 < h2) {
            const int m = (l2 + h2) >> 1;
            if (src[a0 + m] > src[a1 + kk - 1 - m]) l2 = m + 1; else h2 = m;
          }
          const int ai = l2, bi = kk - l2;
          const bool take_a = bi >= lb || (ai < la && src[a0 + ai] > src[a1 + bi]);
          dst[p] = take_a ? src[a0 + ai] : src[a1 + bi];
        }
        for (int i = tid; i <= Rn; i += nt) ro_next[i] = i < Rn ? ro[2 * i] : total;
        __syncthreads();
        uint64_t* t = src; src = dst; dst = t;
        int* u = ro; ro = ro_next; ro_next = u;
        R = Rn;
      }
      gb = src;
      obuf = dst;
    }
    g = min(B, total);
    theta = (g == B) ? gb[B - 1] : 0ull;
    dmax = d;
  }
  __syncthreads();
  keys = gb;

  // ---- flatten: slot of every node, parent slots, outputs, ancestor mask
  // level-local index of every node within its depth, depths 1..dmax at
  // once: per chunk of 64 positions one ballot per depth (every count
  // written, zeros included); then one wave, a lane per depth, turns the
  // counts into per-chunk prefixes and the depths' offsets; then every node
  // takes its depth-major position and writes itself into the inverse table
  {
    const int nchunk = (g + kWave - 1) / kWave;
    for (int c = wid; c < nchunk; c += nt / kWave) {
      const int q = c * kWave + lane;
      const int dq = q < g ? key_depth(keys[q]) : 0;
      for (int dd = 1; dd <= dmax; ++dd) {
        const uint64_t bal = __ballot(dq == dd);
        if (lane == 0) wcnt[c * 34 + dd] = __popcll(bal);
        if (dq == dd) slot_tab[q] = __popcll(bal & lanemask_lt());
      }
    }
    __syncthreads();
    if (tid < kWave) {
      int run = 0;
      if (tid >= 1 && tid <= dmax) {
        for (int c = 0; c < nchunk; ++c) {
          const int t = wcnt[c * 34 + tid];
          wcnt[c * 34 + tid] = run;
          run += t;
        }
      }
      const int inc = wave_inclusive_scan(run);
      if (tid < 34) doff[tid] = inc - run;
    }
    __syncthreads();
    for (int q = tid; q < g; q += nt) {
      const int dq = key_depth(keys[q]);
      roff[doff[dq] + wcnt[(q / kWave) * 34 + dq] + slot_tab[q]] = q + 1;
    }
    __syncthreads();
  }
  if (tid == 0) par_slot[0] = -1;
  for (int q = tid; q < g; q += nt) {
    const uint64_t kq = keys[q];
    const int dq = key_depth(kq);
    const int pl = key_pr(kq) >> 7;
    const int ti = dq == 1 ? -1 : doff[dq - 1] + pl;
    par_slot[q + 1] = (ti >= 0 && ti < g) ? roff[ti] : 0;
  }
  __syncthreads();

  const int64_t ob = (int64_t)r * n_max;
  for (int s = tid; s < n_max; s += nt) {
    int tok, par, dep;
    float sc;
    if (s == 0) {
      tok = root_token[r];
      par = -1;
      dep = 0;
      sc = 0.f;
    } else if (s <= g) {
      const uint64_t kq = keys[s - 1];
      dep = key_depth(kq);
      const int rank = key_pr(kq) & 127;
      tok = ids[((int64_t)r * L + dep - 1) * K + rank];
      par = par_slot[s];
      sc = key_score(kq);
    } else {
      tok = par = dep = -1;
      sc = -INFINITY;
    }
    tok_out[ob + s] = tok;
    par_out[ob + s] = par;
    dep_out[ob + s] = dep;
    if (score_out != nullptr) score_out[ob + s] = sc;
  }
  if (tid == 0) n_nodes_out[r] = g + 1;
  // ancestor masks in two passes.  First every word of every row, word
  // index fastest (whole rows stored in order), with the bits that need no
  // walk: the root's and the row's own.  Then, after a barrier orders the
  // stores, one thread per row walks up from its parent once and rewrites
  // each word that holds an intermediate ancestor (parents precede
  // children, so the walk visits words in non-increasing order and reaches
  // the root in <= L steps).
  const float inv_w = 1.0f / (float)W;
  for (int idx = tid; idx < n_max * W; idx += nt) {
    int s = (int)((float)idx * inv_w);  // idx < 2^24: exact after the fix-up
    if (s * W > idx) --s;
    if ((s + 1) * W <= idx) ++s;
    const int w = idx - s * W;
    uint64_t word = 0;
    if (s <= g) {
      if (w == 0) word = 1ull;
      if ((s >> 6) == w) word |= 1ull << (s & 63);
    }
    mask_out[ob * W + idx] = word;
  }
  __syncthreads();
  for (int s = 1 + tid; s <= g; s += nt) {
    uint64_t* mrow = mask_out + (ob + s) * W;
    const int sw = s >> 6;
    const uint64_t sbit = 1ull << (s & 63);
    int a = par_slot[s];
    int cw = -1;
    uint64_t acc = 0;
    for (int step = 0; step < L && a > 0 && a < s; ++step) {
      const int wa = a >> 6;
      if (wa != cw) {
        if (cw >= 0) mrow[cw] = acc | (cw == 0 ? 1ull : 0ull) | (cw == sw ? sbit : 0ull);
        cw = wa;
        acc = 0;
      }
      acc |= 1ull << (a & 63);
      const int pa = par_slot[a];
      if (pa >= a) break;
      a = pa;
    }
    if (cw >= 0) mrow[cw] = acc | (cw == 0 ? 1ull : 0ull) | (cw == sw ? sbit : 0ull);
  }
}

}  // namespace

hipError_t launch_tree(const float* logp, const int32_t* ids, const int32_t* root, int batch,
                       int L, int k, int k_tree, int budget, int32_t* n_nodes,
                       int32_t* token, int32_t* parent, int32_t* depth, float* score,
                       uint64_t* mask, hipStream_t stream) {
  const TreeLayout lay = tree_layout(L, k_tree, budget);
  // enough threads for one merge element per thread at the common sizes
  int threads = 256;
  while (threads < 1024 && threads < lay.cand_cap) threads <<= 1;
  if (lay.bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(tree_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.bytes);
  hipLaunchKernelGGL(tree_kernel, dim3(batch), dim3(threads), lay.bytes, stream, logp, ids,
                     root, L, k, k_tree, budget, lay.cand_cap, n_nodes, token, parent, depth,
                     score, mask);
  return hipGetLastError();
}

}  // namespace ddt
