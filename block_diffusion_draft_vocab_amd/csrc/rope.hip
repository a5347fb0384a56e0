// Tree positions, rotary embedding and the tree K/V scatter: the step
// between the tree build and verify attention.
//
// [DDTree] "방법론 자세히 보기" (method in detail): the tree is flattened and
// checked by the target in one pass.  A tree token continues the sequence
// after its ancestors only, so the token at depth d sits at sequence position
// P + d (P committed tokens; the root, the bonus token, is at P), whatever its
// slot in the flattened order; a chain reduces to the ordinary positions
// P, P+1, ...  The pages say nothing about the positional encoding itself;
// this is the rotary form with pairs (j, j + D/2) and angle
// position * base^(-2j/D).
//
// One workgroup per (request, tree slot).  The D/2 angles of the slot's
// position are evaluated once, in double precision, into LDS.  Threads own 8
// rotary pairs of one head (a 16-byte piece from each half of the head
// vector) of q or of the new k; the rotation is evaluated in double
// precision, then rounded to float and to bf16 (round to nearest even each
// time).  Other threads copy v.  q is rotated in place; the rotated k and the
// v row go to cache row kv_base + P + slot.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
  return (double)__uint_as_float((uint32_t)b << 16);
}

// float -> bf16, round to nearest even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// Rotates the 8 pairs (lo[e], hi[e]) at pair indices j0 .. j0+7 with the
// (cos, sin) of their angles from cs.
__device__ __forceinline__ void rotate8(u32x4& lo, u32x4& hi, int j0, const double2* cs) {
  u32x4 olo, ohi;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint16_t rl[2], rh[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const double2 a = cs[j0 + e + u];
      const double x = bf16_to_f64(half_of(lo, e + u));
      const double y = bf16_to_f64(half_of(hi, e + u));
      rl[u] = f32_to_bf16((float)(x * a.x - y * a.y));
      rh[u] = f32_to_bf16((float)(y * a.x + x * a.y));
    }
    olo[e >> 1] = (uint32_t)rl[0] | ((uint32_t)rl[1] << 16);
    ohi[e >> 1] = (uint32_t)rh[0] | ((uint32_t)rh[1] << 16);
  }
  lo = olo;
  hi = ohi;
}

__global__ __launch_bounds__(kRopeThreads) void tree_rope_kv_kernel(
    const int32_t* __restrict__ depth, const int32_t* __restrict__ n_nodes, int n_max,
    const int32_t* __restrict__ prefix_len, const int64_t* __restrict__ kv_base, uint16_t* q,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* k_cache,
    uint16_t* v_cache, int hq, int hkv, int D, double base, int32_t* positions) {
  const int slot = blockIdx.x;
  const int r = blockIdx.y;
  const int64_t row = (int64_t)r * n_max + slot;
  int n = n_nodes[r];
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  const bool live = slot < n;
  const int P = prefix_len[r];
  const int pos = live ? P + depth[row] : -1;
  if (positions != nullptr && threadIdx.x == 0) positions[row] = pos;
  if (!live) return;

  // (cos, sin) of the D/2 angles of this position, shared by every head
  __shared__ double2 cs[kRopeMaxD / 2];
  for (int j = threadIdx.x; j < D / 2; j += kRopeThreads) {
    double sn, cn;
    sincos((double)pos * pow(base, -2.0 * j / D), &sn, &cn);
    cs[j] = make_double2(cn, sn);
  }
  __syncthreads();
  const int half_pieces = D / 16;  // 16-byte pieces per half head
  const int rot_items = (hq + hkv) * half_pieces;
  const int copy_items = hkv * (D / 8);
  const int64_t dst_row = kv_base[r] + P + slot;
  for (int it = threadIdx.x; it < rot_items + copy_items; it += kRopeThreads) {
    if (it < rot_items) {
      const int h = it / half_pieces;  // q heads first, then k heads
      const int c = it % half_pieces;
      const bool is_q = h < hq;
      const uint16_t* src = is_q ? q + (row * hq + h) * D : k_new + (row * hkv + (h - hq)) * D;
      u32x4 lo = *reinterpret_cast<const u32x4*>(src + 8 * c);
      u32x4 hi = *reinterpret_cast<const u32x4*>(src + D / 2 + 8 * c);
      rotate8(lo, hi, 8 * c, cs);
      uint16_t* dst = is_q ? q + (row * hq + h) * D : k_cache + (dst_row * hkv + (h - hq)) * D;
      *reinterpret_cast<u32x4*>(dst + 8 * c) = lo;
      *reinterpret_cast<u32x4*>(dst + D / 2 + 8 * c) = hi;
    } else {
      const int i = it - rot_items;  // 16-byte piece of the v row
      *reinterpret_cast<u32x4*>(v_cache + dst_row * hkv * D + 8 * i) =
          *reinterpret_cast<const u32x4*>(v_new + row * hkv * D + 8 * i);
    }
  }
}

}  // namespace

hipError_t launch_tree_rope_kv(const int32_t* depth, const int32_t* n_nodes, int batch, int n_max,
                               const int32_t* prefix_len, const int64_t* kv_base, void* q,
                               const void* k_new, const void* v_new, void* k_cache,
                               void* v_cache, int hq, int hkv, int head_dim, float rope_base,
                               int32_t* positions, hipStream_t stream) {
  hipLaunchKernelGGL(tree_rope_kv_kernel, dim3(n_max, batch), dim3(kRopeThreads), 0, stream,
                     depth, n_nodes, n_max, prefix_len, kv_base, static_cast<uint16_t*>(q),
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), hq, hkv,
                     head_dim, (double)rope_base, positions);
  return hipGetLastError();
}

}  // namespace ddt
