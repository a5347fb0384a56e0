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
//     children (j, rank) with key > theta and (j+1)(rank+1) <= B
//     G := top B of (G u children) by one bitonic sort; theta := G[B-1]
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
  int sort_cap;
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
  int cap = 2;
  const long need = (long)B + nc_bound(B, k_tree);
  while (cap < need) cap <<= 1;
  const int Bp = B > 0 ? B : 1;
  size_t bytes = (size_t)cap * 8 + (size_t)L * k_tree * 4 + (size_t)Bp * 4 * 3 +
                 (size_t)(Bp + 1) * 4 + 34 * 4 * 2 + 18 * 4 + 4 * 4;
  return {cap, bytes};
}

size_t tree_smem_bytes(int L, int k_tree, int budget) {
  return tree_layout(L, k_tree, budget).bytes;
}

namespace {

__global__ __launch_bounds__(1024) void tree_kernel(
    const float* __restrict__ logp, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ root_token, int L, int K, int k_tree, int B, int sort_cap,
    int32_t* __restrict__ n_nodes_out, int32_t* __restrict__ tok_out,
    int32_t* __restrict__ par_out, int32_t* __restrict__ dep_out,
    float* __restrict__ score_out, uint64_t* __restrict__ mask_out) {
  extern __shared__ uint64_t smem_u64[];
  const int Bp = B > 0 ? B : 1;
  uint64_t* keys = smem_u64;
  float* y = reinterpret_cast<float*>(keys + sort_cap);
  float* pscore = y + L * k_tree;
  int* ibuf = reinterpret_cast<int*>(pscore + Bp);
  int* slot_tab = ibuf + Bp;
  int* par_slot = slot_tab + Bp;
  int* dcount = par_slot + Bp + 1;
  int* doff = dcount + 34;
  int* scratch = doff + 34;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int n_max = B + 1;
  const int W = (n_max + 63) / 64;

  for (int i = tid; i < L * k_tree; i += nt) {
    const int d = i / k_tree;
    const int rk = i - d * k_tree;
    y[i] = logp[((int64_t)r * L + d) * K + rk];
  }
  __syncthreads();
  int g = min(k_tree, B);
  for (int i = tid; i < g; i += nt) keys[i] = tkey(y[i], 1, 0, i);
  __syncthreads();
  uint64_t theta = (g == B && B > 0) ? keys[B - 1] : 0ull;

  for (int d = 2; d <= L && g > 0; ++d) {
    // parents: depth d-1 members of G, numbered in G order
    for (int q = tid; q < g; q += nt) ibuf[q] = key_depth(keys[q]) == d - 1;
    __syncthreads();
    const int n = block_scan_array(ibuf, g, scratch);
    if (n == 0) break;
    for (int q = tid; q < g; q += nt) {
      const uint64_t kq = keys[q];
      if (key_depth(kq) == d - 1) pscore[ibuf[q]] = key_score(kq);
    }
    __syncthreads();
    // number of children of each parent that can still enter the top B
    const float* yd = y + (d - 1) * k_tree;
    for (int j = tid; j < n; j += nt) {
      const float s = pscore[j];
      const int cmax = min(k_tree, B / (j + 1));
      int c = 0;
      for (; c < cmax; ++c) {
        const float sc = s + yd[c];
        if (tkey(sc, d, j, c) <= theta) break;
      }
      ibuf[j] = c;
    }
    __syncthreads();
    const int nc = block_scan_array(ibuf, n, scratch);
    if (nc == 0) break;
    for (int j = tid; j < n; j += nt) {
      const int off = ibuf[j];
      const int cnt = (j + 1 < n ? ibuf[j + 1] : nc) - off;
      const float s = pscore[j];
      for (int c = 0; c < cnt; ++c) keys[g + off + c] = tkey(s + yd[c], d, j, c);
    }
    int M = 2;
    while (M < g + nc) M <<= 1;
    for (int i = g + nc + tid; i < M; i += nt) keys[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(keys, M);
    g = min(B, g + nc);
    theta = (g == B) ? keys[B - 1] : 0ull;
  }

  // ---- flatten: slot of every node, parent slots, outputs, ancestor mask
  if (tid < 34) dcount[tid] = 0;
  __syncthreads();
  for (int q = tid; q < g; q += nt) atomicAdd(&dcount[key_depth(keys[q])], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int dd = 0; dd < 34; ++dd) {
      doff[dd] = run;
      run += dcount[dd];
    }
  }
  __syncthreads();
  for (int dd = 1; dd <= L; ++dd) {
    if (dcount[dd] == 0) continue;
    for (int q = tid; q < g; q += nt) ibuf[q] = key_depth(keys[q]) == dd;
    __syncthreads();
    block_scan_array(ibuf, g, scratch);
    for (int q = tid; q < g; q += nt)
      if (key_depth(keys[q]) == dd) slot_tab[doff[dd] + ibuf[q]] = q + 1;
    __syncthreads();
  }
  if (tid == 0) par_slot[0] = -1;
  for (int q = tid; q < g; q += nt) {
    const uint64_t kq = keys[q];
    const int dq = key_depth(kq);
    const int pl = key_pr(kq) >> 7;
    const int ti = dq == 1 ? -1 : doff[dq - 1] + pl;
    par_slot[q + 1] = (ti >= 0 && ti < g) ? slot_tab[ti] : 0;
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
  for (int idx = tid; idx < n_max * W; idx += nt) {
    const int s = idx / W;
    const int w = idx - s * W;
    uint64_t word = 0;
    if (s <= g) {
      // parents precede children, so the walk reaches the root in <= L steps
      int a = s;
      for (int step = 0; step <= L; ++step) {
        if ((a >> 6) == w) word |= 1ull << (a & 63);
        if (a <= 0) break;
        const int pa = par_slot[a];
        if (pa < 0 || pa >= a) break;
        a = pa;
      }
    }
    mask_out[ob * W + idx] = word;
  }
}

}  // namespace

hipError_t launch_tree(const float* logp, const int32_t* ids, const int32_t* root, int batch,
                       int L, int k, int k_tree, int budget, int32_t* n_nodes,
                       int32_t* token, int32_t* parent, int32_t* depth, float* score,
                       uint64_t* mask, hipStream_t stream) {
  const TreeLayout lay = tree_layout(L, k_tree, budget);
  const int threads = lay.sort_cap >= 2048 ? 1024 : (lay.sort_cap >= 1024 ? 512 : 256);
  if (lay.bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(tree_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.bytes);
  hipLaunchKernelGGL(tree_kernel, dim3(batch), dim3(threads), lay.bytes, stream, logp, ids,
                     root, L, k, k_tree, budget, lay.sort_cap, n_nodes, token, parent, depth,
                     score, mask);
  return hipGetLastError();
}

}  // namespace ddt
