// Fused LM head: logits = H . W^T on bf16 MFMA, reduced in the same kernel to
// per-chunk log-sum-exp partials and top-K keys; the top-K merge finishes.
//
// [DFlash] "임베딩과 출력 헤드는 공유한다" (embedding and output head are
// shared): the drafter reuses the target's frozen LM head, so the per-position
// distributions the tree is built from come from one GEMM of the drafter's
// block hidden states with that head.  Fusing the GEMM with the log-softmax /
// top-K pass removes the logits' round trip through HBM: only the weight is
// streamed, once.
//
// Design (HBM-bound on the weight, V x hidden bf16):
//   lmhead_partial  grid (chunks, row blocks of 16), 512 threads (8 waves).
//                   The 16 hidden-state rows sit in LDS (row pad 16 B).  A
//                   chunk is 8 x 16 x kTPW vocab columns; wave w owns the
//                   16-column tiles w, w+8, ... and streams their weight rows
//                   straight into registers with 16-byte loads, one step of
//                   128 hidden units ahead (double buffer), 64 contiguous
//                   bytes of 16 weight rows per load instruction, on
//                   v_mfma_f32_16x16x32_bf16.  The fp32 logits of the chunk are then
//                   staged in LDS (over the hidden rows) and each wave
//                   reduces two rows: max, sum of exp, and the exact top-K
//                   keys (threshold = K-th largest lane maximum, ballot
//                   gather, rank by counting), written in the top-K pass's
//                   partial layout.
//   merge           the top-K merge of the logit pass, over the chunks.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kWavesLm = kLmThreads / kWave;  // 8
constexpr int kStep = 128;                    // hidden units per pipeline step
constexpr int kRowPadBytes = 16;
constexpr int kLmCandCap = 256;  // keys >= T ranked per row in LDS
constexpr float kLog2eLm = 1.4426950408889634f;

__device__ __forceinline__ uint64_t lm_key(float x, int id) {
  return ((uint64_t)f32_order(x + 0.0f) << 32) | (uint64_t)(~(uint32_t)id);  // -0 ties +0
}

__device__ __forceinline__ bf16x8 lds_b128_lm(uint32_t a) {
  return *(const LDS_AS bf16x8*)(uintptr_t)a;
}

// Plain loads: a non-temporal hint made the same pattern 60% slower here.
__device__ __forceinline__ bf16x8 load_w16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <int TPW>
__global__ __launch_bounds__(kLmThreads) void lmhead_partial_kernel(
    const uint16_t* __restrict__ hs, const uint16_t* __restrict__ w, int n_rows, int hidden,
    int vocab, int k, float inv_t, int n_chunks, uint64_t* __restrict__ part_key,
    float2* __restrict__ part_ms) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lm_smem[];
  constexpr int kChunk = kWavesLm * 16 * TPW;  // vocab columns per chunk
  const int chunk = blockIdx.x;
  const int rb = blockIdx.y;  // block of 16 hidden-state rows
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int g = lane >> 4;   // lane group: reduction sub-range / output rows 4g..4g+3
  const int nn = lane & 15;  // A row (hidden-state row) / B column (vocab row)
  const int c0 = chunk * kChunk;
  const int row_stride = hidden * 2 + kRowPadBytes;  // bytes per staged hidden row
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS void*)lm_smem;

  // ---- stage the 16 hidden-state rows (rows past n_rows are zero)
  {
    const int per_row = hidden / 8;  // 16-byte pieces
    for (int i = tid; i < 16 * per_row; i += kLmThreads) {
      const int r = i / per_row, c = i % per_row;
      const int gr = rb * 16 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gr < n_rows) v = *reinterpret_cast<const u32x4*>(hs + (int64_t)gr * hidden + c * 8);
      *(LDS_AS u32x4*)(uintptr_t)(lds0 + r * row_stride + c * 16) = v;
    }
  }

  // ---- this lane's weight rows (one per tile; rows past the vocab read the
  // last row and their results are never used)
  const uint16_t* wrow[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    int v = c0 + 16 * (wid + kWavesLm * t) + nn;
    v = v < vocab ? v : vocab - 1;
    wrow[t] = w + (int64_t)v * hidden + 8 * g;
  }
  // MFMA j of a step covers hidden units [h0 + 32 j, h0 + 32 j + 32); lane
  // group g holds 8 consecutive ones, so one load instruction reads 64
  // contiguous bytes of each of 16 weight rows
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 b0[TPW][4], b1[TPW][4];
  auto load_step = [&](bf16x8 (&b)[TPW][4], int h0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) b[t][j] = load_w16(wrow[t] + h0 + 32 * j);
  };
  const uint32_t a_base = lds0 + nn * row_stride + 16 * g;
  auto mma_step = [&](const bf16x8 (&b)[TPW][4], int h0) {
    bf16x8 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = lds_b128_lm(a_base + h0 * 2 + 64 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[t][j], acc[t], 0, 0, 0);
  };
  const int n_steps = hidden / kStep;  // hidden is a multiple of 2 * kStep
  load_step(b0, 0);
  __syncthreads();  // hidden rows staged
  for (int s = 0; s < n_steps; s += 2) {
    load_step(b1, (s + 1) * kStep);
    mma_step(b0, s * kStep);
    if (s + 2 < n_steps) load_step(b0, (s + 2) * kStep);
    mma_step(b1, (s + 1) * kStep);
  }

  // ---- stage x = fl32(z * inv_t) for the chunk over the hidden rows
  // (lane holds rows 4g..4g+3 of column nn of each tile)
  constexpr int kXStride = kChunk + 4;  // floats per staged logit row
  __syncthreads();
  float* xs = reinterpret_cast<float*>(lm_smem);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int col = 16 * (wid + kWavesLm * t) + nn;
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[(4 * g + i) * kXStride + col] = acc[t][i] * inv_t;
  }
  __syncthreads();

  // ---- per row: (max, sum of exp) and the chunk's top-K keys; wave w
  // reduces rows 2w and 2w+1.  Lane l holds columns l + 64 m.
  constexpr int kPer = (kChunk + kWave - 1) / kWave;
  const int cv = min(kChunk, vocab - c0);  // valid columns of this chunk
  uint32_t* lmax = reinterpret_cast<uint32_t*>(lm_smem + 16 * kXStride * 4) + wid * kWave;
  uint64_t* cand = reinterpret_cast<uint64_t*>(lm_smem + 16 * kXStride * 4 + kLmThreads * 4) +
                   wid * kLmCandCap;
  for (int rr = 0; rr < 2; ++rr) {
    const int r = 2 * wid + rr;
    const int gr = rb * 16 + r;
    if (gr >= n_rows) break;
    const float* xr = xs + r * kXStride;
    float x[kPer];
    float tm = -INFINITY;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int c = lane + kWave * m;
      x[m] = c < cv ? xr[c] : -INFINITY;
      tm = fmaxf(tm, x[m]);
    }
    const float M = wave_max_f(tm);
    float sl = 0.f;
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      sl += (x[m] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((x[m] - M) * kLog2eLm);
    const float S = wave_sum_f(sl);
    // T = the k-th largest lane maximum: k lanes hold a key >= T, so the
    // keys >= T include the chunk's top k (every key when fewer are valid)
    const bool has = tm != -INFINITY;
    lmax[lane] = has ? f32_order(tm) : 0u;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t me = has ? f32_order(tm) : 0u;
    int cnt = 0;
    const u32x4* lm4 = reinterpret_cast<const u32x4*>(lmax);
#pragma unroll
    for (int q = 0; q < kWave / 4; ++q) {
      const u32x4 v = lm4[q];
      cnt += (v.x >= me) + (v.y >= me) + (v.z >= me) + (v.w >= me);
    }
    const uint32_t tsel = wave_max_u32(has && cnt >= k ? me : 0u);
    const float tf = tsel == 0u ? -3.402823466e38f : f32_unorder(tsel);
    // gather the keys >= T (wave-aggregated positions)
    int base = 0;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const bool take = x[m] >= tf;  // -inf (invalid) never passes
      const uint64_t bal = __ballot(take);
      if (take) {
        const int pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (pos < kLmCandCap) cand[pos] = lm_key(x[m], c0 + lane + kWave * m);
      }
      base += __popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int nc = base;
    uint64_t* out = part_key + ((int64_t)gr * n_chunks + chunk) * k;
    if (nc <= kLmCandCap) {
      for (int t = lane; t < nc; t += kWave) {
        const uint64_t v = cand[t];
        // rank = number of greater candidates, two per 16-byte LDS broadcast
        int rank = 0;
        const u32x4* c2 = reinterpret_cast<const u32x4*>(cand);
        for (int u = 0; u < nc / 2; ++u) {
          const u32x4 q = c2[u];
          rank += (((uint64_t)q.y << 32 | q.x) > v) + (((uint64_t)q.w << 32 | q.z) > v);
        }
        if (nc & 1) rank += cand[nc - 1] > v;
        if (rank < k) out[rank] = v;
      }
      for (int j = nc + lane; j < k; j += kWave) out[j] = 0ull;
    } else {
      // massive ties: k rounds of a wave arg-max below the previous key
      uint64_t prev = ~0ull;
      for (int j = 0; j < k; ++j) {
        uint64_t b = 0;
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
          const int c = lane + kWave * m;
          const uint64_t key = c < cv ? lm_key(x[m], c0 + c) : 0ull;
          if (key < prev && key > b) b = key;
        }
#pragma unroll
        for (int d = kWave / 2; d > 0; d >>= 1) {
          const uint64_t o = shfl_xor_u64(b, d);
          b = o > b ? o : b;
        }
        prev = b;
        if (lane == 0) out[j] = b;
      }
    }
    if (lane == 0) part_ms[(int64_t)gr * n_chunks + chunk] = make_float2(M, S);
  }
}

}  // namespace

int lmhead_chunks(int vocab) { return (vocab + kLmChunk - 1) / kLmChunk; }

size_t lmhead_smem_bytes(int hidden) {
  const size_t rows = 16 * ((size_t)hidden * 2 + kRowPadBytes);
  const size_t red = 16 * (size_t)(kLmChunk + 4) * 4 + kLmThreads * 4 +
                     (size_t)kWavesLm * kLmCandCap * 8;
  return rows > red ? rows : red;
}

size_t lmhead_workspace_bytes(int n_rows, int vocab, int k) {
  const size_t nc = lmhead_chunks(vocab);
  return ((size_t)n_rows * nc * k * sizeof(uint64_t) + 255) / 256 * 256 +
         (size_t)n_rows * nc * sizeof(float2);
}

hipError_t launch_lmhead_topk(const void* hs, const void* w, int n_rows, int hidden, int vocab,
                              int k, float inv_t, int32_t* ids, float* logp, float* lse,
                              void* ws, hipStream_t stream) {
  const int nc = lmhead_chunks(vocab);
  uint64_t* part_key = static_cast<uint64_t*>(ws);
  float2* part_ms = reinterpret_cast<float2*>(
      static_cast<char*>(ws) + ((size_t)n_rows * nc * k * sizeof(uint64_t) + 255) / 256 * 256);
  const size_t smem = lmhead_smem_bytes(hidden);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(lmhead_partial_kernel<kLmTilesPerWave>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(lmhead_partial_kernel<kLmTilesPerWave>, dim3(nc, (n_rows + 15) / 16),
                     dim3(kLmThreads), smem, stream, static_cast<const uint16_t*>(hs),
                     static_cast<const uint16_t*>(w), n_rows, hidden, vocab, k, inv_t, nc,
                     part_key, part_ms);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(part_key, part_ms, n_rows, nc, k, ids, logp, lse, stream);
}

}  // namespace ddt
