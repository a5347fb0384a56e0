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
//   mask bits.  A workgroup has 8 waves (two per SIMD, so one wave's softmax
//   overlaps the other's MFMAs); wave w owns the 32 columns [32w, 32w+32) of
//   the workgroup's 256 and every wave walks the same 64-key tiles.
//   The 1-D grid enumerates (KV head, request, column group, key split) with
//   the KV head fastest: workgroups are dealt to the 8 XCDs round-robin, so
//   with 8 KV heads all workgroups of one head share an XCD and its L2.  A
//   trailing column group with few columns gets fewer key splits and is
//   enumerated beside the full groups of the same split.  A second
//   kernel merges the splits with their log-sum-exp weights.
//
// Per 64-key tile
//   staging: K and V rows are copied global -> LDS by the load unit itself
//     (global_load_lds_dwordx4, no registers involved), the 16-byte chunks
//     of each row XOR-swizzled against bank conflicts (one swizzle for the
//     K reads, another for the transposing V reads); a ring of three tiles
//     keeps the copies two tiles ahead, one barrier per tile.
//   S^T (keys x cols) = K . Q^T     v_mfma_f32_32x32x16_bf16, two 32-key
//     halves = two independent accumulation chains.  Each lane then holds 16
//     keys of ONE column per half, so a row reduction needs one exchange
//     with lane^32 (v_permlane32_swap).
//   O^T (D x cols) += V^T . P^T     P straight from the S^T registers (keys
//     relabelled inside each 16-key chunk), V^T fragments read from the
//     row-major V tile with the transposing ds_read_b64_tr_b16.
// Visibility is applied per key from a 64-bit window of the column's mask
// row, computed for all own-row tiles of the split before the tile loop and
// kept in LDS; tiles no column of the workgroup can see are skipped.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
#define LDS_AS __attribute__((address_space(3)))

constexpr int kKT = 64;  // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kColsPerWave = 32;
constexpr int kColsPerWG = kWaves * kColsPerWave;
constexpr int kRing = 3;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;
constexpr int kMaxTilesPerSplit = 16;
constexpr int kMinTilesPerSplit = 3;  // measured: 2 and 4 were slower for one 256-column group
constexpr int kCUs = 256;
constexpr int kXcds = 8;  // accelerator dies; consecutive workgroups go to different ones

template <int D>
struct Geo {
  static constexpr int kCh = D / 8;                        // 16-byte chunks per key row
  static constexpr int kRowBytes = D * 2;
  // Physical 16-byte chunk of logical chunk c in tile row r is c ^ swz(r).
  // K: the sixteen lanes a ds_read_b128 serves together read one logical
  // chunk of sixteen consecutive rows, which must land in sixteen different
  // bank groups.  V: a ds_read_b64_tr_b16 lane group reads two adjacent
  // chunks of four consecutive rows, which must land in eight different
  // bank groups.  (Measured: 284 and 129 B/clk per CU, the instructions'
  // full rates, against 164 and 84 with a plain row & 7 swizzle.)
  static __device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (r & 15) : (D == 64 ? ((r >> 1) & 7) : (r & 3));
  }
  static __device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? 2 * (r & 3) : (D == 64 ? (r & 2) : (r & 3));
  }
  static constexpr int kTileBytes = kKT * kRowBytes;       // one K or V tile
  static constexpr int kLoads = 2 * kKT * kCh / kThreads;  // 16-byte copies per thread per tile
  static constexpr int kSmem = 2 * kRing * kTileBytes;     // K ring, then V ring
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
  uint16_t* part_o;   // bf16 [rows][n_split][D], normalised by the split's own sum
  float2* part_ml;    // [rows][n_split] = (max in log2 units, sum of 2^(x - max))
  int batch, hq, hkv, n_q_max, mask_words;
  int n_cg_full;      // column groups with all 8 waves busy at n_q_max
  int n_split;        // key splits of those groups
  int n_split_tail;   // key splits of the trailing partial group (0: none)
  int max_tiles;      // key tiles of the longest request the plan was made for
  int block_len;      // > 0: own rows form blocks of this many rows, each query
                      // sees only its own block's rows (packed drafter blocks)
  int g;              // q-heads per KV head
  float scale_log2;
  // the launch's fixed divisors, as multiply-and-shift pairs
  FastDiv fd_groups;  // column groups per (request, KV head, split)
  FastDiv fd_msplit;  // max(n_split, n_split_tail)
  FastDiv fd_hkv, fd_hq, fd_g, fd_nq_max;
  FastDiv fd_tiles;   // max_tiles
  FastDiv fd_split, fd_split_tail;
  FastDiv fd_block;   // block_len (1 without packed blocks)
};

// Tiles [t0, t1) of split s out of n_split over nt tiles (balanced; 32-bit
// products: n_split <= 2^15 and nt < 2^16 under the plan's limits).
// Tiles [t0, t1) of split s: nt / n_split each, the remainder one apiece to
// the first splits.  Those are dispatched first, and the last split, which
// holds the own rows (and their visibility setup), stays among the short ones.
__device__ __forceinline__ void split_range(int s, int n_split, int nt, int& t0, int& t1,
                                            const Params& p) {
  // the plan's split counts divide through their multipliers; a count
  // scaled down for a shorter request through the float estimate
  const int q = n_split == (int)p.fd_split.d         ? fdiv(nt, p.fd_split)
                : n_split == (int)p.fd_split_tail.d  ? fdiv(nt, p.fd_split_tail)
                : nt < (1 << 21)                     ? div_small(nt, n_split)
                                                     : (int)((unsigned)nt / (unsigned)n_split);
  const int rem = nt - q * n_split;
  t0 = s * q + (s < rem ? s : rem);
  t1 = t0 + q + (s < rem ? 1 : 0);
}
// Key splits request r actually uses: the plan's count scaled by the
// request's share of the longest key range, so that a short request in a
// ragged batch gets splits of about the same length as the longest one
// (never more tiles per split than the plan allows: ns >= max_tiles / 16).
__device__ __forceinline__ int request_splits(int ns, int nt, const Params& p) {
  const int max_tiles = p.max_tiles;
  if (nt >= max_tiles) return ns;
  // below 2^16 tiles the plan keeps ns <= 4096, so the rounded-up product
  // stays under 2^31 and divides through the multiplier
  const long v = max_tiles <= 0xFFFF ? (long)fdiv(nt * ns + max_tiles - 1, p.fd_tiles)
                                     : ((long)nt * ns + max_tiles - 1) / max_tiles;
  return v < 1 ? 1 : (v > ns ? ns : (int)v);
}
// Split s is empty only when there are fewer tiles than splits.
__device__ __forceinline__ bool split_nonempty(int s, int n_split, int nt, const Params& p) {
  if (nt >= n_split) return true;
  int t0, t1;
  split_range(s, n_split, nt, t0, t1, p);
  return t0 < t1;
}

// Words j0>>6 and (j0>>6)+1 of a mask row of W words (word 0 and nothing
// when j0 < 0), zero past the row.
__device__ __forceinline__ void mask_words_for(const uint64_t* mrow, int W, int j0, uint64_t& lo,
                                               uint64_t& hi) {
  const int w = j0 < 0 ? 0 : (j0 >> 6);
  lo = w < W ? mrow[w] : 0ull;
  hi = (j0 >= 0 && w + 1 < W) ? mrow[w + 1] : 0ull;
}

// Which of the 64 keys [key0, key0+64) a column may see: all prefix keys,
// and own keys j in [own_lo, own_hi) that its mask row allows (all of them
// without a mask).  lo/hi come from mask_words_for(key0 - P); key0 + 64 > P - 64.
__device__ __forceinline__ uint64_t visible64(int key0, int P, int own_lo, int own_hi,
                                              bool has_mask, uint64_t lo, uint64_t hi) {
  if (key0 + kKT <= P) return ~0ull;
  const uint64_t pre = key0 >= P ? 0ull : ((1ull << (P - key0)) - 1ull);
  const int j0 = key0 - P;
  int b_lo = own_lo - j0;
  b_lo = b_lo < 0 ? 0 : b_lo;
  int b_hi = own_hi - j0;
  b_hi = b_hi > 64 ? 64 : b_hi;
  uint64_t range = 0ull;
  if (b_hi > b_lo)
    range = (b_hi >= 64 ? ~0ull : ((1ull << b_hi) - 1ull)) & ~((1ull << b_lo) - 1ull);
  uint64_t own = ~0ull;
  if (has_mask) {
    const int sh = j0 & 63;
    own = j0 < 0 ? (lo << (-j0)) : (sh ? ((lo >> sh) | (hi << (64 - sh))) : lo);
  }
  return pre | (own & range);
}

// x combined with the value of lane ^ 32 (same column, other key half).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The V^T fragments of one 16-key chunk: 2R ds_read_b64_tr_b16 and their
// wait, in one asm statement.  (The compiler's intrinsic makes every use wait
// for all LDS-direct copies in flight, including the ones for later tiles;
// in inline asm a read left in flight past its statement could land in a
// register the compiler has already reused, so each statement waits for its
// own reads.)  Fragment dt reads columns 32 dt of rows R0 / R1 from base
// va0 (even dt) or va1 (odd dt), the second pair of fragments 128 bytes on.
// Outputs are early-clobber: no read may overwrite an address register
// before a later read of the statement has used it.
template <int R, int R0, int R1>
__device__ __forceinline__ void lds_tr_chunk(uint32_t va0, uint32_t va1, i16x4 (&t)[R][2]) {
  if constexpr (R == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1]), "=&v"(t[2][0]),
          "=&v"(t[2][1]), "=&v"(t[3][0]), "=&v"(t[3][1])
        : "v"(va0), "v"(va1), "i"(R0), "i"(R1), "i"(R0 + 128), "i"(R1 + 128));
  } else if constexpr (R == 2) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1])
        : "v"(va0), "v"(va1), "i"(R0), "i"(R1));
  } else {
    static_assert(R == 1, "head_dim");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0][0]), "=&v"(t[0][1])
        : "v"(va0), "i"(R0), "i"(R1));
  }
}
__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t a) {
  return *(const LDS_AS bf16x8*)(uintptr_t)a;
}

template <int N>
struct IntC {
  static constexpr int value = N;
};
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (expcnt / lgkmcnt fields left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// Stores of split partials with device scope (sc1): they write through the
// XCD's L2, so no dirty partial lines are left for the write-back at the end
// of the kernel (measured: the merge kernel starts 2.6-3.3 us earlier after
// a budget-256 verify launch, whose partials are ~15 MB).  The merge kernel
// is their only reader.
__device__ __forceinline__ void store_partial16(void* ptr, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(ptr), "v"(v) : "memory");
}
__device__ __forceinline__ void store_partial8(void* ptr, float2 v) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  const f2 w = {v.x, v.y};
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(ptr), "v"(w) : "memory");
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(Params p) {
  using G = Geo<D>;
  // Every parameter is read here, before the first branch.  Left alone, the
  // compiler sinks each scalar load to its first use behind the early exits,
  // and a workgroup pays one scalar round trip per use before its first tile
  // copy.  (Input operands only: the pointers keep their address space.)
  asm volatile("" ::"s"(p.q), "s"(p.k), "s"(p.v), "s"(p.kv_base), "s"(p.prefix_len), "s"(p.n_q));
  asm volatile("" ::"s"(p.mask), "s"(p.out), "s"(p.lse), "s"(p.part_o), "s"(p.part_ml));
  asm volatile("" ::"s"(p.batch), "s"(p.hq), "s"(p.hkv), "s"(p.n_q_max), "s"(p.mask_words),
               "s"(p.n_cg_full), "s"(p.n_split), "s"(p.n_split_tail), "s"(p.max_tiles),
               "s"(p.block_len), "s"(p.g), "s"(p.scale_log2));
  asm volatile("" ::"s"(p.fd_groups.m), "s"(p.fd_groups.s), "s"(p.fd_msplit.m),
               "s"(p.fd_msplit.s), "s"(p.fd_hkv.m), "s"(p.fd_hkv.s), "s"(p.fd_g.m), "s"(p.fd_g.s),
               "s"(p.fd_tiles.m), "s"(p.fd_tiles.s), "s"(p.fd_split.m), "s"(p.fd_split.s));
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  __shared__ int tile_list[kMaxTilesPerSplit];
  __shared__ int n_tiles_s;
  __shared__ uint32_t own_need[kMaxTilesPerSplit];
  __shared__ uint64_t win_lds[kMaxTilesPerSplit][kColsPerWG];  // own-row tile windows
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int h2 = lane >> 5;
  const int n = lane & 31;

  // ---- decode the work item.  Workgroups are dealt round-robin to the 8
  // XCDs (blockIdx % 8), each XCD starting its share in blockIdx order.
  // The column groups of one (split, KV head, request) read the same K/V
  // tiles, so they are made consecutive in one XCD's dispatch order: they
  // run side by side and each tile comes from HBM once into that XCD's L2.
  // The triples themselves go round-robin over the XCDs.  One request: KV
  // head fastest, so with 8 KV heads each XCD holds one head and every
  // split of a column group finds that group's Q rows in its L2 (measured:
  // split fastest instead made the budget-256 verify launch 27 -> 39 us).
  // Several requests: split fastest, so the splits of one request land on
  // different XCDs and every XCD gets a similar mix of long and short
  // requests (ragged serving batch 327 -> 303 us per step stage).
  const int max_split = p.n_split > p.n_split_tail ? p.n_split : p.n_split_tail;
  const int xcd = blockIdx.x % kXcds;
  const int jx = blockIdx.x / kXcds;
  int cg;
  int x = fdivmod(jx, p.fd_groups, cg) * kXcds + xcd;
  int s, hk, r;
  if (p.batch == 1) {
    r = 0;
    s = fdivmod(x, p.fd_hkv, hk);
    if (s >= max_split) return;  // padding of the last round
  } else {
    x = fdivmod(x, p.fd_msplit, s);
    r = fdivmod(x, p.fd_hkv, hk);
    if (r >= p.batch) return;  // padding of the last round
  }
  int n_split = cg < p.n_cg_full ? p.n_split : p.n_split_tail;

  // the request's sizes and cache base: three loads, one round trip
  const int P = p.prefix_len[r];
  const int nq_req = p.n_q[r];
  const int64_t base = p.kv_base[r];
  asm volatile("" ::"s"(P), "s"(nq_req), "s"(base));
  const int nq = min(nq_req, p.n_q_max);
  const int T = P + nq;
  const int g = p.g;
  const int ncols = nq * g;
  const int col0 = cg * kColsPerWG;
  if (col0 >= ncols || T <= 0) return;
  const int ntiles = (T + kKT - 1) / kKT;
  n_split = request_splits(n_split, ntiles, p);
  if (s >= n_split) return;
  int t_begin, t_end;
  split_range(s, n_split, ntiles, t_begin, t_end, p);
  if (t_begin >= t_end) return;
  // a split spans at most kMaxTilesPerSplit tiles whenever every request's
  // prefix_len + n_q is within the max_kv_len the plan was made for; the
  // clamp only keeps a violated bound from indexing past the tile list
  if (t_end - t_begin > kMaxTilesPerSplit) t_end = t_begin + kMaxTilesPerSplit;
  const bool wave_active = col0 + wid * kColsPerWave < ncols;
  const bool has_mask = p.mask != nullptr;

  // ---- this lane's column
  const int col = col0 + wid * kColsPerWave + n;
  const bool valid = col < ncols;
  int col_h;
  const int col_q = fdivmod(col, p.fd_g, col_h);
  const int qi = valid ? col_q : 0;
  const int head = hk * g + (valid ? col_h : 0);
  const uint64_t* mrow =
      has_mask ? p.mask + ((int64_t)r * p.n_q_max + qi) * p.mask_words : nullptr;
  const bool lane_mask = has_mask && valid;
  // own rows this column may see: all nq, or its packed block
  const int own_lo = p.block_len > 0 ? fdiv(qi, p.fd_block) * p.block_len : 0;
  const int own_hi = p.block_len > 0 ? min(nq, own_lo + p.block_len) : nq;

  // ---- staging: copy j of this thread moves 16-byte chunk
  // L = (8 j + wid) * 64 + lane of the (K tile | V tile) pair; a wave's 64
  // chunks are contiguous in LDS, which is what the LDS-direct load writes.
  // Copies j < kLoads/2 are K chunks, the rest V (with one copy per thread,
  // waves 0-3 copy K and waves 4-7 V).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS void*)smem_raw;
  const int row_stride = p.hkv * D;  // elements; a request's rows span < 2^31 elements
  const uint16_t* kbase = p.k + base * row_stride + (int64_t)hk * D;
  const uint16_t* vbase = p.v + base * row_stride + (int64_t)hk * D;
  // The per-thread part of each copy's address is the same for every tile
  // and computed here once: a tile's copies then cost one scalar base each,
  // plus a clamp of the rows past the request's last key in its final tile.
  int ld_row[G::kLoads];
  int ld_col[G::kLoads];       // element offset of the logical chunk
  uint32_t ld_off[G::kLoads];  // byte offset of the copy inside a whole tile
  uint32_t ld_lds[G::kLoads];  // wave-uniform LDS offset inside one slot pair
  constexpr int kPer = kKT * G::kCh;
#pragma unroll
  for (int j = 0; j < G::kLoads; ++j) {
    const int L = (8 * j + wid) * 64 + lane;
    const bool isv = G::kLoads == 1 ? wid >= 4 : j >= G::kLoads / 2;
    const int Lt = isv ? L - kPer : L;
    ld_row[j] = Lt / G::kCh;
    ld_col[j] = ((Lt % G::kCh) ^ (isv ? G::swz_v(ld_row[j]) : G::swz_k(ld_row[j]))) * 8;
    ld_off[j] = (uint32_t)(ld_row[j] * row_stride + ld_col[j]) * 2u;
    ld_lds[j] = __builtin_amdgcn_readfirstlane((Lt - lane) * 16) +
                (isv ? kRing * G::kTileBytes : 0);
  }
  auto issue_tile = [&](int t, int slot) {
    const int key0 = t * kKT;
    const uint32_t slot_lds = lds0 + slot * G::kTileBytes;
    if (key0 + kKT <= T) {
#pragma unroll
      for (int j = 0; j < G::kLoads; ++j) {
        const bool isv = G::kLoads == 1 ? wid >= 4 : j >= G::kLoads / 2;
        // (the source goes through a named pointer: passed as an expression,
        // the host compilation pass drops the kernel's launch stub)
        const char* src =
            reinterpret_cast<const char*>((isv ? vbase : kbase) + (int64_t)key0 * row_stride) +
            ld_off[j];
        __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(uintptr_t)(slot_lds + ld_lds[j]), 16,
                                         0, 0);
      }
    } else {
      const int last = T - 1 - key0;  // rows past the end copy a valid row, never visible
#pragma unroll
      for (int j = 0; j < G::kLoads; ++j) {
        const bool isv = G::kLoads == 1 ? wid >= 4 : j >= G::kLoads / 2;
        const uint16_t* tb = (isv ? vbase : kbase) + (int64_t)key0 * row_stride;
        const int row = ld_row[j] < last ? ld_row[j] : last;
        const uint16_t* src = tb + (row * row_stride + ld_col[j]);
        __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)(uintptr_t)(slot_lds + ld_lds[j]), 16,
                                         0, 0);
      }
    }
  };

  // Q, then the split's first tile, are put in flight before the tile list
  // is built.  Prefix tiles are always processed; a range that starts in the
  // own rows is copied speculatively and re-copied below in the rare case
  // that the list skips that tile.
  // (waves without a column of the request load no Q: in a drafter block six
  // of the eight waves are idle, and their Q rows would take the CU's fill
  // bandwidth ahead of the first tile)
  bf16x8 qf[D / 16];
  if (wave_active) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(
        p.q + (((int64_t)r * p.n_q_max + qi) * p.hq + head) * D + 8 * h2);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = qp[2 * t];
  } else {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = bf16x8{};
  }
  __builtin_amdgcn_sched_barrier(0);  // the Q loads stay ahead of the tile copies
  issue_tile(t_begin, 0);

  // ---- tiles to process: every tile holding prefix keys, and the own-row
  // tiles in which some column of the workgroup sees a key.  The visibility
  // windows of the range's own-row tiles are computed here once (their mask
  // words loaded together: one memory latency) and kept in LDS, so the tile
  // loop issues no memory operation besides the tile copies.
  // Without a mask or packed blocks every own key is visible to every
  // column: no tile is skipped and the loop derives its windows from P and nq.
  const int nt_range = t_end - t_begin;
  const bool listed = (has_mask || p.block_len > 0) && t_end * kKT > P;
  int ntl = nt_range;
  if (listed) {
    for (int i = tid; i < nt_range; i += kThreads) own_need[i] = 0u;
    uint64_t wlo[kMaxTilesPerSplit], whi[kMaxTilesPerSplit];
#pragma unroll
    for (int i = 0; i < kMaxTilesPerSplit; ++i) {
      wlo[i] = whi[i] = 0ull;
      const int key0 = (t_begin + i) * kKT;
      if (i < nt_range && key0 + kKT > P && lane_mask)
        mask_words_for(mrow, p.mask_words, key0 - P, wlo[i], whi[i]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxTilesPerSplit; ++i) {
      const int key0 = (t_begin + i) * kKT;
      if (i >= nt_range || key0 + kKT <= P) continue;
      const uint64_t w =
          valid ? visible64(key0, P, own_lo, own_hi, has_mask, wlo[i], whi[i]) : 0ull;
      if (h2 == 0) win_lds[i][wid * kColsPerWave + n] = w;
      if (wave_active && __ballot(w != 0ull) != 0 && lane == 0) atomicOr(&own_need[i], 1u);
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
  auto tile_at = [&](int i) {
    return listed ? __builtin_amdgcn_readfirstlane(tile_list[i]) : t_begin + i;
  };

  // ---- per-lane LDS read offsets inside one slot.
  // K as the A operand of S^T: row n (+32 for the second half), logical
  // chunk 2tt + h2, physical chunk (2tt) ^ (h2 ^ swz_k(n)).
  uint32_t koff[D / 16];
  {
    const int w = h2 ^ G::swz_k(n);  // rows n and n + 32 share the swizzle
#pragma unroll
    for (int tt = 0; tt < D / 16; ++tt)
      koff[tt] = (uint32_t)(n * G::kRowBytes + (((2 * tt) ^ w) * 16));
  }
  // V^T through the transposing read: the address lane (q4 = lane/16, e,
  // rr) names row (q4/2)*4 + e (+8 for the second read of a pair, +16 per
  // key chunk) and columns 32 dt + 16 (q4 & 1) + 4 rr, whose physical chunk
  // is (4 dt) ^ z; the read hands lane l column l%32 of 4 rows, which is the
  // A-operand layout with key slots matching the P^T registers.
  uint32_t voff[2];
  {
    const int q4 = lane >> 4, e = (lane >> 2) & 3, rr = lane & 3;
    const int row = (q4 >> 1) * 4 + e;
    const int y = (q4 & 1) * 2 + (rr >> 1);
    const int z = y ^ G::swz_v(row);  // unchanged by the +8 / +16 row offsets
#pragma unroll
    for (int u = 0; u < 2; ++u)
      voff[u] = (uint32_t)(row * G::kRowBytes + (((4 * u) ^ z) * 16) + (rr & 1) * 8);
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};

  // prologue: if the list does not start with the speculated tile, let
  // that copy land and copy the right one.  Then Q and tile 0 are waited
  // for, and only then is tile 1 copied: the compiler, which cannot order
  // the Q loads against the LDS-direct copies, waits for every copy in
  // flight before the first use of Q, and each CU takes its Q rows and
  // tiles at 64 B per clock, so a tile 1 issued earlier would delay the
  // first tile by its own transfer.  Inside the loop the only memory
  // operations in flight are tile copies, so "all but the newest tile" is
  // a plain vmcnt.
  if (ntl > 0 && tile_at(0) != t_begin) {
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // every wave's speculative copy has landed
    __asm__ volatile("" ::: "memory");
    issue_tile(tile_at(0), 0);
  }
  wait_vm<0>();
  // columns past the end (loaded from row 0 of the request) are zeroed
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    if (!valid) qf[t] = bf16x8{};
  if (ntl > 1) issue_tile(tile_at(1), 1);

  for (int i = 0; i < ntl; ++i) {
    // this tile's copies done (the next tile's may stay in flight), then
    // the barrier publishes it and retires the slot read at i - 1
    if (i + 1 < ntl) wait_vm<G::kLoads>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    const int ti = tile_at(i);
    if (i + 2 < ntl) issue_tile(tile_at(i + 2), (i + 2) % kRing);
    if (!wave_active) continue;
    const int key0 = ti * kKT;

    const int slot = i % kRing;
    const uint32_t kb = lds0 + slot * G::kTileBytes;
    const uint32_t vb = lds0 + (kRing + slot) * G::kTileBytes;
    // all K fragments of the tile are read up front (32 reads in flight
    // instead of a read -> wait -> MFMA chain)
    bf16x8 ka[D / 16], kb2[D / 16];
#pragma unroll
    for (int tt = 0; tt < D / 16; ++tt) {
      ka[tt] = lds_b128(kb + koff[tt]);
      kb2[tt] = lds_b128(kb + koff[tt] + 32 * G::kRowBytes);
    }
    f32x16 sa = f32x16{}, sb = f32x16{};
#pragma unroll
    for (int tt = 0; tt < D / 16; ++tt) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[tt], qf[tt], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb2[tt], qf[tt], sb, 0, 0, 0);
    }
    // keep the scheduler from sinking the reads back between the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, D / 8, 0);  // the K reads
    __builtin_amdgcn_sched_group_barrier(0x008, D / 8, 0);  // then the MFMAs
    float xv[32];
    if (key0 + kKT <= P) {  // tile inside the prefix: every key visible
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        xv[v] = sa[v];
        xv[16 + v] = sb[v];
      }
    } else {
      const uint64_t win =
          (listed ? win_lds[ti - t_begin][wid * kColsPerWave + n]
                  : (valid ? visible64(key0, P, 0, nq, false, 0ull, 0ull) : 0ull)) >>
          (4 * h2);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = (v >> 2) * 8 + (v & 3);
        xv[v] = ((win >> kk) & 1ull) ? sa[v] : -INFINITY;
        xv[16 + v] = ((win >> (32 + kk)) & 1ull) ? sb[v] : -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 32; ++v) tmax = fmaxf(tmax, xv[v]);
    tmax = xor32_max(tmax) * p.scale_log2;
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
    bf16x8 pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[c][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(xv[8 * c + e], p.scale_log2, neg_m));
    }
    // row sum of the bf16 weights the P.V product actually uses
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pf[c][e], pf[c][e + 1]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls, false);
      }
    }
    l_run += ls;
    const uint32_t va0 = vb + voff[0], va1 = vb + voff[1];
    // V^T fragments of key chunk c (tile rows [16c, 16c+16)), then its
    // MFMAs; those run while the next chunk's reads are waited for
    static_for<4>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      constexpr int r0 = 16 * c * G::kRowBytes, r1 = r0 + 8 * G::kRowBytes;
      i16x4 tv[D / 32][2];
      lds_tr_chunk<D / 32, r0, r1>(va0, va1, tv);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(tv[dt][0], tv[dt][1]), pf[c], o[dt],
                                                        0, 0, 0);
    });
  }
  // ---- result rows (bf16): the output itself without splits, else this
  // split's partial, normalised by its own sum.  The O^T fragments scatter
  // 8-byte pieces over 32 rows, so each wave first transposes its 32 rows
  // through LDS (the tile ring is free once every wave is past the loop)
  // and then writes whole rows with 16-byte stores.
  constexpr int kRowPad = D * 2 + 16;  // bytes per staged row (pad: bank spread)
  __syncthreads();
  if (!wave_active) return;
  const float l_tot = xor32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const uint32_t stage = lds0 + wid * (kColsPerWave * kRowPad);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = dt * 32 + a * 8 + h2 * 4;
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        h[e] = __builtin_bit_cast(uint16_t, (__bf16)(o[dt][a * 4 + e] * inv));
      typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
      const u32x2 w = {(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                       (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
      *(LDS_AS u32x2*)(uintptr_t)(stage + n * kRowPad + d0 * 2) = w;
    }
  }
  if (valid && h2 == 0) {
    const int64_t rowid = ((int64_t)r * p.n_q_max + qi) * p.hq + head;
    if constexpr (SPLIT) {
      store_partial8(p.part_ml + rowid * p.n_split + s, make_float2(m_run, l_tot));
    } else {
      if (p.lse != nullptr)
        p.lse[rowid] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // D/8 lanes per row, 64 / (D/8) rows per instruction.  The element offset
  // of the row a lane stores is stepped from one division up front (with a
  // division per store, the address arithmetic rather than the stores set
  // the time of this loop), and every staged row is read before the stores.
  constexpr int kLpr = D / 8;
  constexpr int kRpi = 64 / kLpr;
  const int chunk = lane % kLpr;
  u32x4 rv[kColsPerWave / kRpi];
#pragma unroll
  for (int rr = 0; rr < kColsPerWave; rr += kRpi)
    rv[rr / kRpi] =
        *(const LDS_AS u32x4*)(uintptr_t)(stage + (rr + lane / kLpr) * kRowPad + chunk * 16);
  const int cfirst = col0 + wid * kColsPerWave + lane / kLpr;
  int ho;
  const int q0 = fdivmod(cfirst, p.fd_g, ho);
  const int dq = fdiv(kRpi, p.fd_g), dh = kRpi - dq * g;
  const int64_t ostride = SPLIT ? (int64_t)p.n_split * D : (int64_t)D;  // elements per row id
  int64_t eoff = (((int64_t)r * p.n_q_max + q0) * p.hq + hk * g + ho) * ostride +
                 (SPLIT ? (int64_t)s * D : 0) + chunk * 8;
  const int64_t step = (int64_t)(dq * p.hq + dh) * ostride;
  const int64_t wrap = (int64_t)(p.hq - g) * ostride;
#pragma unroll
  for (int rr = 0; rr < kColsPerWave; rr += kRpi) {
    if (cfirst + rr < ncols) {
      if constexpr (SPLIT) store_partial16(p.part_o + eoff, rv[rr / kRpi]);
      else *reinterpret_cast<u32x4*>(p.out + eoff) = rv[rr / kRpi];
    }
    eoff += step;
    ho += dh;
    if (ho >= g) {
      ho -= g;
      eoff += wrap;
    }
  }
}

// Merge of the key splits: one group of D/8 threads per (request, query
// row, q-head), each thread owning 8 consecutive output elements (16-byte
// partial loads and stores).  Splits are read kBatch at a time with all
// 2 * kBatch loads in flight, merged into a running (max, weighted sum) like
// the tile loop.  With one request (kSpec), whose length the plan was sized
// for, and a plan of at most kBatch splits, every slot is loaded in one
// batch before the request's sizes arrive: slot indexes are clamped to the
// plan's split count for the row's column group (inside the row's stride, so
// every load is unconditional and in bounds), and the slots the request
// leaves empty or repeats are masked once the sizes are known, so the launch
// waits on one round trip of loads instead of two.  A batch of requests of
// mixed lengths loads only the slots each request fills, a batch at a time.
template <int D, int kBatch, bool kSpec>
__global__ __launch_bounds__(256) void attn_combine_kernel(Params p) {
  constexpr int kTPR = D / 8;
  const int gid = blockIdx.x * (int)(blockDim.x / kTPR) + threadIdx.x / kTPR;
  const int lane = threadIdx.x % kTPR;
  if (gid >= p.batch * p.n_q_max * p.hq) return;
  int head, qi;
  const int rq = fdivmod(gid, p.fd_hq, head);
  const int r = fdivmod(rq, p.fd_nq_max, qi);
  const int g = p.g;
  int head_in;
  (void)fdivmod(head, p.fd_g, head_in);
  const int col = qi * g + head_in;
  const int ns_plan = col / kColsPerWG < p.n_cg_full ? p.n_split : p.n_split_tail;
  const int64_t ro = (int64_t)gid * p.n_split;
  const int nq_r = p.n_q[r];
  const int prefix_r = p.prefix_len[r];
  float M = -INFINITY;
  float Lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // one batch of slots into the running (M, Lsum, acc)
  auto merge = [&](const float2* ml, const u32x4* raw) {
    float bm = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) bm = fmaxf(bm, ml[u].x);
    if (bm == -INFINITY) return;
    const float alpha = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - bm);
    Lsum *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    M = bm;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = ml[u].x == -INFINITY ? 0.f : ml[u].y * __builtin_amdgcn_exp2f(ml[u].x - M);
      Lsum += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * __uint_as_float(raw[u][e] << 16);
        acc[2 * e + 1] += w * __uint_as_float(raw[u][e] & 0xFFFF0000u);
      }
    }
  };
  bool live;
  if constexpr (kSpec) {
    // the launch gives kBatch >= every split count of the plan: one batch
    float2 ml[kBatch];
    u32x4 raw[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int su = u < ns_plan ? u : (ns_plan > 0 ? ns_plan - 1 : 0);
      ml[u] = p.part_ml[ro + su];
      raw[u] = *reinterpret_cast<const u32x4*>(p.part_o + (ro + su) * D + lane * 8);
    }
    // every load above is issued before the first use of the sizes waits
    __builtin_amdgcn_sched_barrier(0);
    const int nq = min(nq_r, p.n_q_max);
    const int T = prefix_r + nq;
    live = qi < nq && T > 0;
    const int ntiles = (T + kKT - 1) / kKT;
    const int ns = live ? request_splits(ns_plan, ntiles, p) : 0;
    // slots past the request's splits (repeats included) or left empty
    if (ns < kBatch || ntiles < ns) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (!(u < ns && split_nonempty(u, ns, ntiles, p))) {
          ml[u] = make_float2(-INFINITY, 0.f);
          raw[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if (live) merge(ml, raw);
  } else {
    const int nq = min(nq_r, p.n_q_max);
    const int T = prefix_r + nq;
    live = qi < nq && T > 0;
    const int ntiles = (T + kKT - 1) / kKT;
    const int ns = live ? request_splits(ns_plan, ntiles, p) : 0;
    for (int sp0 = 0; sp0 < ns; sp0 += kBatch) {
      float2 ml[kBatch];
      u32x4 raw[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int sp = sp0 + u;
        const bool ok = sp < ns && split_nonempty(sp, ns, ntiles, p);
        ml[u] = ok ? p.part_ml[ro + sp] : make_float2(-INFINITY, 0.f);
        raw[u] = ok ? *reinterpret_cast<const u32x4*>(p.part_o + (ro + sp) * D + lane * 8)
                    : u32x4{0u, 0u, 0u, 0u};
      }
      merge(ml, raw);
    }
  }
  if (!live) return;
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  u32x4 wv;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    wv[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2 * e] * inv)) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2 * e + 1] * inv)) << 16);
  *reinterpret_cast<u32x4*>(p.out + (int64_t)gid * D + lane * 8) = wv;
  if (lane == 0 && p.lse != nullptr)
    p.lse[gid] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

bool plan_splits(const AttnPlan& plan) { return plan.n_split > 1 || plan.n_split_tail > 1; }

template <int D>
hipError_t launch_d(const Params& prm, const AttnPlan& plan, hipStream_t stream) {
  const int n_groups = plan.n_cg_full + (plan.n_split_tail > 0 ? 1 : 0);
  const int max_split = plan.n_split > plan.n_split_tail ? plan.n_split : plan.n_split_tail;
  // (head, request, split) triples in rounds of kXcds, times the column groups
  const long triples = (long)max_split * prm.batch * prm.hkv;
  const int wgs = (int)(((triples + kXcds - 1) / kXcds) * kXcds * n_groups);
  constexpr size_t smem = Geo<D>::kSmem;
  if (wgs <= 0) return hipSuccess;
  if (plan_splits(plan)) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<D, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL((attn_kernel<D, true>), dim3(wgs), dim3(kThreads), smem, stream, prm);
    // 256-thread workgroups, or 64 when that leaves most CUs idle (a
    // drafter block's few rows: every CU then holds some of the loads)
    const int rows = prm.batch * prm.n_q_max * prm.hq;
    const int threads = (long)rows * (D / 8) < 256L * kCUs ? 64 : 256;
    const int rpb = threads / (D / 8);
    // 8 slots per batch when the plan has at most 8 splits (fewer repeated
    // or empty slots), else 16; a single request's plan in one batch
    const dim3 grid((rows + rpb - 1) / rpb);
    if (prm.batch == 1 && max_split <= 16) {
      if (max_split <= 8)
        hipLaunchKernelGGL((attn_combine_kernel<D, 8, true>), grid, dim3(threads), 0, stream,
                           prm);
      else
        hipLaunchKernelGGL((attn_combine_kernel<D, 16, true>), grid, dim3(threads), 0, stream,
                           prm);
    } else {
      if (max_split <= 8)
        hipLaunchKernelGGL((attn_combine_kernel<D, 8, false>), grid, dim3(threads), 0, stream,
                           prm);
      else
        hipLaunchKernelGGL((attn_combine_kernel<D, 16, false>), grid, dim3(threads), 0, stream,
                           prm);
    }
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<D, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL((attn_kernel<D, false>), dim3(wgs), dim3(kThreads), smem, stream, prm);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

AttnPlan attn_plan(int batch, int hq, int hkv, int n_q_max, int max_kv_len) {
  const int g = hq / hkv;
  const int cols = n_q_max * g;
  const int n_cg_full = cols / kColsPerWG;
  const int tail_waves = (cols % kColsPerWG + kColsPerWave - 1) / kColsPerWave;
  const int max_tiles = (max_kv_len + kKT - 1) / kKT;
  const int min_split = (max_tiles + kMaxTilesPerSplit - 1) / kMaxTilesPerSplit;
  const long heavy = (long)batch * hkv * n_cg_full;
  const long tail = tail_waves > 0 ? (long)batch * hkv : 0;
  // One workgroup per CU (the LDS ring holds one): split the full column
  // groups as far as the CUs allow, the trailing partial group in proportion
  // to its busy waves (a lone wave runs a tile in about half the time eight
  // waves take: copies and barriers do not shrink with it).
  auto clamp_split = [&](long v) {
    if (v < min_split) v = min_split;
    if (v > max_tiles) v = max_tiles;
    return (int)(v < 1 ? 1 : v);
  };
  auto tail_split = [&](int s) {
    if (tail_waves == 0) return 0;
    const int t = (s * tail_waves + 1) / 2;
    return clamp_split(t > s ? s : t);
  };
  AttnPlan plan;
  plan.n_cg_full = n_cg_full;
  if (heavy > 0) {
    long s = kCUs / heavy;
    // at least kMinTilesPerSplit tiles per split: a split of one or two
    // tiles costs more in partial stores and merge reads than it saves
    const long by_tiles = max_tiles / kMinTilesPerSplit;
    if (s > by_tiles) s = by_tiles;
    while (s > 1 && heavy * s + tail * tail_split((int)s) > kCUs) --s;
    plan.n_split = clamp_split(s);
    // Several requests decode split fastest over the XCDs (a workgroup's XCD
    // is its triple index mod 8): an even split count would tie split s to
    // the XCDs of its residue, and since a short request leaves its last
    // splits empty, those XCDs would idle while the first ones queue the
    // long requests' work (measured: a ragged batch at 8 splits took 1.5x
    // its 9-split time).  An odd count walks every split over every XCD.
    if (batch > 1 && plan.n_split % 2 == 0 && plan.n_split < max_tiles) ++plan.n_split;
    plan.n_split_tail = tail_split(plan.n_split);
  } else {
    // only a partial group per head (drafter-sized queries): half a
    // workgroup per CU, so every workgroup gets two or more tiles and the
    // split merge has half as many partials to read (measured fastest)
    plan.n_split = clamp_split(kCUs / 2 / (tail > 0 ? tail : 1));
    plan.n_split_tail = tail_waves > 0 ? plan.n_split : 0;
  }
  return plan;
}

size_t attn_workspace_bytes(int batch, int hq, int hkv, int head_dim, int n_q_max,
                            int max_kv_len) {
  const AttnPlan plan = attn_plan(batch, hq, hkv, n_q_max, max_kv_len);
  if (!plan_splits(plan)) return 0;
  const size_t rows = (size_t)batch * n_q_max * hq * plan.n_split;
  return align256(rows * head_dim * sizeof(uint16_t)) + align256(rows * sizeof(float2));
}

hipError_t launch_attention(int batch, int hq, int hkv, int head_dim, int n_q_max,
                            int mask_words, int max_kv_len, float scale, const void* q,
                            const void* k, const void* v, const int64_t* kv_base,
                            const int32_t* prefix_len, const int32_t* n_q,
                            const uint64_t* mask, int block_len, void* out, float* lse, void* ws,
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
  const bool split = plan_splits(plan);
  const size_t rows = (size_t)batch * n_q_max * hq * plan.n_split;
  prm.part_o = split ? static_cast<uint16_t*>(ws) : nullptr;
  prm.part_ml = split ? reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                                  align256(rows * head_dim * sizeof(uint16_t)))
                      : nullptr;
  prm.batch = batch;
  prm.hq = hq;
  prm.hkv = hkv;
  prm.n_q_max = n_q_max;
  prm.mask_words = mask_words;
  prm.n_cg_full = plan.n_cg_full;
  prm.n_split = plan.n_split;
  prm.n_split_tail = plan.n_split_tail;
  prm.block_len = block_len;
  prm.max_tiles = (max_kv_len + kKT - 1) / kKT;
  prm.g = hq / hkv;
  prm.scale_log2 = scale * kLog2e;
  prm.fd_groups = make_fastdiv(plan.n_cg_full + (plan.n_split_tail > 0 ? 1 : 0));
  prm.fd_msplit = make_fastdiv(plan.n_split > plan.n_split_tail ? plan.n_split : plan.n_split_tail);
  prm.fd_hkv = make_fastdiv(hkv);
  prm.fd_hq = make_fastdiv(hq);
  prm.fd_g = make_fastdiv(hq / hkv);
  prm.fd_nq_max = make_fastdiv(n_q_max);
  prm.fd_tiles = make_fastdiv(prm.max_tiles);
  prm.fd_split = make_fastdiv(plan.n_split);
  prm.fd_split_tail = make_fastdiv(plan.n_split_tail);
  prm.fd_block = make_fastdiv(block_len > 0 ? block_len : 1);
  switch (head_dim) {
    case 32: return launch_d<32>(prm, plan, stream);
    case 64: return launch_d<64>(prm, plan, stream);
    case 128: return launch_d<128>(prm, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ddt
