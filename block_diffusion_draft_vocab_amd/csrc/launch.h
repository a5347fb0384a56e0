// Host-side launchers of the libddt kernels (internal; the public ABI is
// include/ddt.h).  Arguments are validated by the ABI layer before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddt {

// ---- stage 1 --------------------------------------------------------------
struct TopkPlan {
  int n_chunks;
  int chunk_len;  // multiple of 4, <= kTopkMaxChunk
};
constexpr int kTopkThreads = 256;
constexpr int kTopkPerThread = 32;
constexpr int kTopkMaxChunk = kTopkThreads * kTopkPerThread;  // 8192
constexpr int kTopkMergeMaxLists = 256;   // chunk lists one merge handles per row
constexpr int kTopkMergeMaxKeys = 16384;  // chunk lists x k
TopkPlan topk_plan(int n_rows, int vocab, int k);
bool topk_supported(int n_rows, int vocab, int k);
size_t topk_workspace_bytes(int n_rows, int vocab, int k);
hipError_t launch_topk(const float* logits, int64_t ld, int n_rows, int vocab, int k,
                       float inv_t, int32_t* ids, float* logp, float* lse, void* ws,
                       hipStream_t stream);
// Device address of the allocation-free top-K entry point's scratch array on
// the current device (looked up once per device, nothing allocated).
hipError_t topk_noalloc_scratch(void** ptr);

// Merge of per-chunk partials (sorted key lists + (max, sum of exp)) into
// the rows' top-k ids / log-probs / lse; shared by the logit pass and the
// fused LM head.  n_chunks <= kTopkMergeMaxLists, n_chunks * k <=
// kTopkMergeMaxKeys.
hipError_t launch_topk_merge(const uint64_t* part_key, const float2* part_ms, int n_rows,
                             int n_chunks, int k, int32_t* ids, float* logp, float* lse,
                             hipStream_t stream);

// ---- fused LM head + log-softmax / top-K --------------------------------
constexpr int kLmThreads = 512;
constexpr int kLmTilesPerWave = 5;                            // 16-column vocab tiles
constexpr int kLmChunk = (kLmThreads / 64) * 16 * kLmTilesPerWave;  // 640 columns
constexpr int kLmMaxK = 64;
int lmhead_chunks(int vocab);
size_t lmhead_smem_bytes(int hidden);
size_t lmhead_workspace_bytes(int n_rows, int vocab, int k);
hipError_t launch_lmhead_topk(const void* hs, const void* w, int n_rows, int hidden, int vocab,
                              int k, float inv_t, int32_t* ids, float* logp, float* lse,
                              void* ws, hipStream_t stream);

// ---- tree positions + rotary embedding + tree K/V scatter -------------------
constexpr int kRopeThreads = 256;
constexpr int kRopeMaxD = 256;
hipError_t launch_tree_rope_kv(const int32_t* depth, const int32_t* n_nodes, int batch, int n_max,
                               const int32_t* prefix_len, const int64_t* kv_base, void* q,
                               const void* k_new, const void* v_new, void* k_cache,
                               void* v_cache, int hq, int hkv, int head_dim, float rope_base,
                               int32_t* positions, hipStream_t stream);

// ---- target argmax (the verifier's greedy tokens) ------------------------
struct ArgmaxPlan {
  int n_chunks;
  int chunk_len;  // multiple of 4, <= kArgmaxMaxChunk
};
constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxPerThread = 32;
constexpr int kArgmaxMaxChunk = kArgmaxThreads * kArgmaxPerThread;  // 8192
constexpr int kArgmaxMaxRows = 65535;  // rows are grid.y
ArgmaxPlan argmax_plan(int n_rows, int vocab);
size_t argmax_workspace_bytes(int n_rows, int vocab);
hipError_t launch_argmax(const float* logits, int64_t ld, int n_rows, int vocab, int32_t* ids,
                         float* maxv, void* ws, hipStream_t stream);

// ---- stage 2 --------------------------------------------------------------
size_t tree_smem_bytes(int L, int k_tree, int budget);
hipError_t launch_tree(const float* logp, const int32_t* ids, const int32_t* root, int batch,
                       int L, int k, int k_tree, int budget, int32_t* n_nodes,
                       int32_t* token, int32_t* parent, int32_t* depth, float* score,
                       uint64_t* mask, hipStream_t stream);

// ---- stage 3 --------------------------------------------------------------
struct AttnPlan {
  int n_cg_full;     // column groups of 256 columns per (request, kv head)
  int n_split;       // key splits of each full group
  int n_split_tail;  // key splits of the trailing partial group (0: none)
};
AttnPlan attn_plan(int batch, int hq, int hkv, int n_q_max, int max_kv_len);
size_t attn_workspace_bytes(int batch, int hq, int hkv, int head_dim, int n_q_max,
                            int max_kv_len);
hipError_t launch_attention(int batch, int hq, int hkv, int head_dim, int n_q_max,
                            int mask_words, int max_kv_len, float scale, const void* q,
                            const void* k, const void* v, const int64_t* kv_base,
                            const int32_t* prefix_len, const int32_t* n_q,
                            const uint64_t* mask, int block_len, void* out, float* lse, void* ws,
                            hipStream_t stream);

// ---- stage 4 --------------------------------------------------------------
hipError_t launch_accept(const int32_t* token, const int32_t* parent, const int32_t* n_nodes,
                         int n_max, const int32_t* target, int batch, int L, void* k_cache,
                         void* v_cache, const int64_t* kv_base, const int32_t* prefix_len,
                         int n_layers, int64_t layer_stride, int hkv, int head_dim,
                         int32_t* accept_len, int32_t* accepted, int32_t* bonus,
                         int32_t* new_len, hipStream_t stream);

}  // namespace ddt
