// Stage 3: masked GQA attention on bf16 MFMA (gfx950).
//
// Verify mode ([DDTree] "방법론 자세히 보기", "용어 정리"): each flattened tree
// token attends to the whole prefix and, among the tree rows, to its ancestor
// path only (bit j of its mask row).  Drafter mode ([DFlash] "DFlash의 핵심
// 아이디어" points 2-3, [DFlash-news] "DFlash 핵심 기술 구조"): block queries
// attend to all injected context rows and to every row of their block.
//
// Work decomposition
//   A "column" is one (query row, q-head) pair of a KV head; the g = hq/hkv
//   q-heads of one query are adjacent columns, so they share K/V tiles and
//   mask bits.  A wave owns 64 columns (two 32-column MFMA blocks), a
//   workgroup of 4 waves owns 256 columns and one range of 32-key tiles.
//   Grid x = (column group, request, KV head) with the KV head fastest, so
//   with 8 KV heads every workgroup of one head lands on the same XCD and
//   its K/V tiles stay in that XCD's L2.  Grid y = key split; a second
//   kernel merges the splits with their log-sum-exp weights.
//
// Per 32-key tile (staged once in LDS for the 4 waves):
//   S^T (keys x cols) = K (32 x D) . Q^T        v_mfma_f32_32x32x16_bf16
//   each lane then holds 16 keys of ONE column, so the softmax row
//   reductions need only one exchange with lane^32;
//   O^T (D x cols) += V^T (D x 32) . P^T        P taken straight from the
//   S^T registers (keys relabelled inside each 16-key chunk; V is written
//   to LDS transposed with the same relabelling).
// Visibility is applied per key from a 32-bit window of the column's mask
// row; tiles no column of a wave can see are skipped.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kKT = 32;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kColsPerWave = 32;
constexpr int kColsPerWG = kWaves * kColsPerWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;
constexpr int kMaxTilesPerSplit = 32;

template <int D>
struct Smem {
  uint16_t k[kKT][D + 8];   // row-major, padded against bank conflicts
  uint16_t vt[D][kKT + 8];  // transposed, keys relabelled per 16-chunk
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int64_t* kv_base;
  const int32_t* prefix_len;
  const int32_t* n_q;
  const uint64_t* mask;
  uint16_t* out;
  float* lse;
  float* part_o;
  float2* part_ml;
  int batch, hq, hkv, n_q_max, mask_words, n_cg, n_split, tps;
  float scale_log2;
};

// Position of key kt (0..31) inside its LDS V^T row: within each 16-key
// chunk keys {0-3, 8-11} come first, then {4-7, 12-15}.  That is the order
// in which a 32x32 accumulator half (lanes 0-31 / 32-63) holds them.
__device__ __forceinline__ int vt_pos(int kt) {
  const int w = kt & 15;
  return (kt & ~15) | (w & 3) | ((w & 4) << 1) | ((w & 8) >> 1);
}

// Bits b in [0, 32) = bit (j0 + b) of a little-endian u64 row of W words,
// zero outside [0, 64 W).  Requires j0 > -32.
__device__ __forceinline__ uint32_t extract32(const uint64_t* row, int W, int j0) {
  const int j = j0 < 0 ? 0 : j0;
  const int w = j >> 6;
  const int sh = j & 63;
  const uint64_t lo = w < W ? row[w] : 0ull;
  const uint64_t hi = (w + 1) < W ? row[w + 1] : 0ull;
  const uint64_t v = sh ? ((lo >> sh) | (hi << (64 - sh))) : lo;
  const uint32_t r = (uint32_t)v;
  return j0 < 0 ? (r << (-j0)) : r;
}

// Which of the 32 keys [key0, key0+32) a column may see.
__device__ __forceinline__ uint32_t visible_window(int key0, int P, int nq, const uint64_t* mrow,
                                                   int W, bool valid) {
  if (!valid) return 0u;
  if (key0 + kKT <= P) return 0xFFFFFFFFu;
  const uint32_t pre = key0 >= P ? 0u : ((1u << (P - key0)) - 1u);
  const int j0 = key0 - P;
  const int lo = j0 < 0 ? -j0 : 0;
  int hi = nq - j0;
  hi = hi > 32 ? 32 : hi;
  uint32_t range = 0u;
  if (hi > lo) range = (hi >= 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u)) & ~((1u << lo) - 1u);
  const uint32_t own = mrow != nullptr ? extract32(mrow, W, j0) : 0xFFFFFFFFu;
  return pre | (own & range);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 8 waves per workgroup, wave w owns the 32 columns [32w, 32w+32) of the
// workgroup's 256 and every wave walks the same tiles (two per SIMD, so one
// wave's softmax overlaps the other's MFMAs).  Tiles sit in a ring of three
// LDS buffers, loaded two tiles ahead, with one barrier per tile.
template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem<D>* sm = reinterpret_cast<Smem<D>*>(smem_raw);   // ring of 3 tiles
  __shared__ int tile_list[kMaxTilesPerSplit];
  __shared__ int n_tiles_s;
  __shared__ uint32_t own_need[kMaxTilesPerSplit];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int h2 = lane >> 5;
  const int n = lane & 31;

  const int x = blockIdx.x;
  const int hk = x % p.hkv;
  const int rest = x / p.hkv;
  const int r = rest % p.batch;
  const int cg = rest / p.batch;
  const int s = blockIdx.y;

  const int P = p.prefix_len[r];
  const int nq = min(p.n_q[r], p.n_q_max);
  const int T = P + nq;
  const int g = p.hq / p.hkv;
  const int ncols = nq * g;
  const int col0 = cg * kColsPerWG;
  if (col0 >= ncols) return;
  const int ntiles = (T + kKT - 1) / kKT;
  const int t_begin = s * p.tps;
  const int t_end = min(ntiles, t_begin + p.tps);
  if (t_begin >= t_end) return;
  const int64_t base = p.kv_base[r];
  const bool wave_active = col0 + wid * kColsPerWave < ncols;

  // ---- this lane's column
  const int col = col0 + wid * kColsPerWave + n;
  const bool valid = col < ncols;
  const int qi = valid ? col / g : 0;
  const int head = hk * g + (valid ? col % g : 0);
  const uint64_t* mrow =
      p.mask != nullptr ? p.mask + ((int64_t)r * p.n_q_max + qi) * p.mask_words : nullptr;

  // ---- tiles to process: every tile holding prefix keys, and the own-row
  // tiles in which some column of the workgroup sees a key
  const int nt_range = t_end - t_begin;
  const bool listed = t_end * kKT > P;
  int ntl = nt_range;
  if (listed) {
    for (int i = tid; i < nt_range; i += kThreads) own_need[i] = 0u;
    __syncthreads();
    if (wave_active) {
      for (int i = 0; i < nt_range; ++i) {
        const int key0 = (t_begin + i) * kKT;
        if (key0 + kKT <= P) continue;
        const uint32_t w = visible_window(key0, P, nq, mrow, p.mask_words, valid);
        if (__ballot(w != 0u) != 0 && lane == 0) atomicOr(&own_need[i], 1u);
      }
    }
    __syncthreads();
    if (tid == 0) {
      int m = 0;
      for (int i = 0; i < nt_range; ++i) {
        const int key0 = (t_begin + i) * kKT;
        if (key0 + kKT <= P || own_need[i] != 0u) tile_list[m++] = t_begin + i;
      }
      n_tiles_s = m;
    }
    __syncthreads();
    ntl = n_tiles_s;
  }
  auto tile_at = [&](int i) { return listed ? tile_list[i] : t_begin + i; };

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};

  // ---- cooperative staging.  Thread = (16-byte chunk of D, key pair) with
  // the key pair fastest, so a transposed V write instruction covers 16
  // consecutive words of one LDS row.
  constexpr int kChunks = D / 8;
  constexpr int kTasks = 16 * kChunks;
  const bool has_task = tid < kTasks;
  const int kp = tid & 15;
  const int dc = (tid >> 4) % kChunks;
  const int64_t row_stride = (int64_t)p.hkv * D;
  const uint16_t* kbase = p.k + base * row_stride + (int64_t)hk * D + dc * 8;
  const uint16_t* vbase = p.v + base * row_stride + (int64_t)hk * D + dc * 8;
  u32x4 rk0{}, rk1{}, rv0{}, rv1{};
  auto load_tile = [&](int t) {
    const int ka = t * kKT + 2 * kp;
    const int64_t off = (int64_t)ka * row_stride;
    const u32x4 z{};
    rk0 = ka < T ? ld16(kbase + off) : z;
    rv0 = ka < T ? ld16(vbase + off) : z;
    rk1 = ka + 1 < T ? ld16(kbase + off + row_stride) : z;
    rv1 = ka + 1 < T ? ld16(vbase + off + row_stride) : z;
  };
  auto store_tile = [&](Smem<D>& b) {
    *reinterpret_cast<u32x4*>(&b.k[2 * kp][dc * 8]) = rk0;
    *reinterpret_cast<u32x4*>(&b.k[2 * kp + 1][dc * 8]) = rk1;
    const int pos = vt_pos(2 * kp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = (rv0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t b2 = (rv1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(&b.vt[dc * 8 + e][pos]) = a | (b2 << 16);
    }
  };

  // prologue: the first two tiles' loads and the Q loads are all in flight
  // together; the ring of three LDS buffers then keeps loads two tiles ahead
  u32x4 pk0{}, pk1{}, pv0{}, pv1{};
  if (has_task && ntl > 0) load_tile(tile_at(0));
  if (has_task && ntl > 1) {
    pk0 = rk0; pk1 = rk1; pv0 = rv0; pv1 = rv1;
    load_tile(tile_at(1));
  }
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = p.q + (((int64_t)r * p.n_q_max + qi) * p.hq + head) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      qf[t] = valid ? *reinterpret_cast<const bf16x8*>(qp + 16 * t + 8 * h2) : bf16x8{};
  }
  if (has_task && ntl > 1) {
    store_tile(sm[1]);
    rk0 = pk0; rk1 = pk1; rv0 = pv0; rv1 = pv1;
  }
  if (has_task && ntl > 0) store_tile(sm[0]);
  __syncthreads();
  if (has_task && ntl > 2) load_tile(tile_at(2));
  for (int i = 0; i < ntl; ++i) {
    if (wave_active) {
      const Smem<D>& b = sm[i % 3];
      const int key0 = tile_at(i) * kKT;
      // two independent accumulation chains (even / odd head-dim steps)
      f32x16 sacc = f32x16{}, sacc1 = f32x16{};
#pragma unroll
      for (int tt = 0; tt < D / 16; tt += 2) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&b.k[n][16 * tt + 8 * h2]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&b.k[n][16 * tt + 16 + 8 * h2]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[tt], sacc, 0, 0, 0);
        sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[tt + 1], sacc1, 0, 0, 0);
      }
      sacc += sacc1;
      float xv[16];
      float tmax = -INFINITY;
      if (key0 + kKT <= P) {  // tile inside the prefix: every key visible
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          xv[v] = sacc[v];
          tmax = fmaxf(tmax, xv[v]);
        }
      } else {
        const uint32_t win = visible_window(key0, P, nq, mrow, p.mask_words, valid);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = (v >> 2) * 8 + h2 * 4 + (v & 3);
          xv[v] = ((win >> kk) & 1u) ? sacc[v] : -INFINITY;
          tmax = fmaxf(tmax, xv[v]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)) * p.scale_log2;
      // Lazy rescaling: the reference max only moves when the tile max
      // exceeds it by more than 2^8, so p = 2^(x - m) stays <= 256 and the
      // O/l rescale (a pass over every accumulator) is rare after the first
      // tile.  O/l does not depend on the reference.
      const bool grow = tmax > m_run + kRescaleLog2;
      if (__ballot(grow) != 0) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float ls = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        xv[v] = __builtin_amdgcn_exp2f(fmaf(xv[v], p.scale_log2, neg_m));
        ls += xv[v];
      }
      l_run += ls;
      bf16x8 pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[c][e] = (__bf16)xv[(2 * c + (e >> 2)) * 4 + (e & 3)];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(&b.vt[dt * 32 + n][16 * c + 8 * h2]);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c], o[dt], 0, 0, 0);
        }
      }
    }
    if (i + 2 < ntl) {
      if (has_task) store_tile(sm[(i + 2) % 3]);  // buffer last read at i - 1
      __syncthreads();
      if (has_task && i + 3 < ntl) load_tile(tile_at(i + 3));
    }
  }
  if (!wave_active) return;

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!valid) return;
  const int64_t rowid = ((int64_t)r * p.n_q_max + qi) * p.hq + head;
  if constexpr (!SPLIT) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = p.out + rowid * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = dt * 32 + a * 8 + h2 * 4;
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          h[e] = __builtin_bit_cast(uint16_t, (__bf16)(o[dt][a * 4 + e] * inv));
        uint2 w;
        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    }
    if (p.lse != nullptr && h2 == 0)
      p.lse[rowid] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t ro = rowid * p.n_split + s;
    float* po = p.part_o + ro * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = dt * 32 + a * 8 + h2 * 4;
        *reinterpret_cast<float4*>(po + d0) = make_float4(
            o[dt][a * 4 + 0], o[dt][a * 4 + 1], o[dt][a * 4 + 2], o[dt][a * 4 + 3]);
      }
    }
    if (h2 == 0) p.part_ml[ro] = make_float2(m_run, l_tot);
  }
}

// Merge of the key splits: one group of D/4 threads per (request, query
// row, q-head), each thread owning 4 consecutive output elements (float4
// partial loads, 8-byte bf16 stores).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(Params p) {
  constexpr int kTPR = D / 4;
  constexpr int kRPB = 256 / kTPR;
  const int gid = blockIdx.x * kRPB + threadIdx.x / kTPR;
  const int lane = threadIdx.x % kTPR;
  if (gid >= p.batch * p.n_q_max * p.hq) return;
  const int rq = gid / p.hq;
  const int qi = rq % p.n_q_max;
  const int r = rq / p.n_q_max;
  const int nq = min(p.n_q[r], p.n_q_max);
  if (qi >= nq) return;
  const int T = p.prefix_len[r] + nq;
  const int ntiles = (T + kKT - 1) / kKT;
  const int ns = min(p.n_split, (ntiles + p.tps - 1) / p.tps);
  const int64_t ro = (int64_t)gid * p.n_split;
  float M = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, p.part_ml[ro + sp].x);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float Lsum = 0.f;
  if (M != -INFINITY) {
    for (int sp = 0; sp < ns; ++sp) {
      const float2 ml = p.part_ml[ro + sp];
      const float w = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
      Lsum += ml.y * w;
      const float4 o4 = *reinterpret_cast<const float4*>(p.part_o + (ro + sp) * D + lane * 4);
      acc.x += o4.x * w;
      acc.y += o4.y * w;
      acc.z += o4.z * w;
      acc.w += o4.w * w;
    }
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  uint2 wv;
  wv.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.x * inv)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.y * inv)) << 16);
  wv.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.z * inv)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc.w * inv)) << 16);
  *reinterpret_cast<uint2*>(p.out + (int64_t)gid * D + lane * 4) = wv;
  if (lane == 0 && p.lse != nullptr)
    p.lse[gid] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const Params& prm, const AttnPlan& plan, hipStream_t stream) {
  const dim3 grid(plan.n_cg * prm.batch * prm.hkv, plan.n_split);
  constexpr size_t smem = 3 * sizeof(Smem<D>);
  if (plan.n_split > 1) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<D, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL((attn_kernel<D, true>), grid, dim3(kThreads), smem, stream, prm);
    const int rows = prm.batch * prm.n_q_max * prm.hq;
    const int rpb = 256 / (D / 4);
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((rows + rpb - 1) / rpb), dim3(256), 0,
                       stream, prm);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<D, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL((attn_kernel<D, false>), grid, dim3(kThreads), smem, stream, prm);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

AttnPlan attn_plan(int batch, int hq, int hkv, int n_q_max, int max_kv_len) {
  const int g = hq / hkv;
  const int n_cg = (n_q_max * g + kColsPerWG - 1) / kColsPerWG;
  const int max_tiles = (max_kv_len + kKT - 1) / kKT;
  // one workgroup per CU where the shape allows it (a second partial round
  // of workgroups would double the time), long prefixes cut to <= 32 tiles
  const long wgs = (long)batch * hkv * n_cg;
  int n_split = (int)(256 / wgs);
  const int by_len = (max_tiles + kMaxTilesPerSplit - 1) / kMaxTilesPerSplit;
  if (by_len > n_split) n_split = by_len;
  if (n_split > max_tiles) n_split = max_tiles;
  if (n_split < 1) n_split = 1;
  const int tps = (max_tiles + n_split - 1) / n_split;
  n_split = (max_tiles + tps - 1) / tps;
  return {n_cg, n_split, tps};
}

size_t attn_workspace_bytes(int batch, int hq, int hkv, int head_dim, int n_q_max,
                            int max_kv_len) {
  const AttnPlan plan = attn_plan(batch, hq, hkv, n_q_max, max_kv_len);
  if (plan.n_split <= 1) return 0;
  const size_t rows = (size_t)batch * n_q_max * hq * plan.n_split;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float2));
}

hipError_t launch_attention(int batch, int hq, int hkv, int head_dim, int n_q_max,
                            int mask_words, int max_kv_len, float scale, const void* q,
                            const void* k, const void* v, const int64_t* kv_base,
                            const int32_t* prefix_len, const int32_t* n_q,
                            const uint64_t* mask, void* out, float* lse, void* ws,
                            hipStream_t stream) {
  const AttnPlan plan = attn_plan(batch, hq, hkv, n_q_max, max_kv_len);
  Params prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.kv_base = kv_base;
  prm.prefix_len = prefix_len;
  prm.n_q = n_q;
  prm.mask = mask;
  prm.out = static_cast<uint16_t*>(out);
  prm.lse = lse;
  const size_t rows = (size_t)batch * n_q_max * hq * plan.n_split;
  prm.part_o = static_cast<float*>(ws);
  prm.part_ml = plan.n_split > 1 ? reinterpret_cast<float2*>(
                                       static_cast<char*>(ws) +
                                       align256(rows * head_dim * sizeof(float)))
                                 : nullptr;
  prm.batch = batch;
  prm.hq = hq;
  prm.hkv = hkv;
  prm.n_q_max = n_q_max;
  prm.mask_words = mask_words;
  prm.n_cg = plan.n_cg;
  prm.n_split = plan.n_split;
  prm.tps = plan.tiles_per_split;
  prm.scale_log2 = scale * kLog2e;
  switch (head_dim) {
    case 32: return launch_d<32>(prm, plan, stream);
    case 64: return launch_d<64>(prm, plan, stream);
    case 128: return launch_d<128>(prm, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ddt
