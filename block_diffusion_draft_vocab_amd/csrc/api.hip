// C ABI of libddt: argument validation on the host, then the launches.
// Every entry point returns a status code; nothing is enqueued on error.
#include <math.h>

#include <cstdint>

#include "../../include/ddt.h"
#include "launch.h"

#define DDT_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? DDT_OK : DDT_ELAUNCH; }

}  // namespace

DDT_EXPORT int ddt_abi_version(void) { return DDT_ABI_VERSION; }

DDT_EXPORT const char* ddt_status_string(int status) {
  switch (status) {
    case DDT_OK: return "ok";
    case DDT_EINVAL: return "invalid argument";
    case DDT_EUNSUPPORTED: return "unsupported shape";
    case DDT_EWORKSPACE: return "workspace too small";
    case DDT_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

// ---- stage 1 ---------------------------------------------------------------
static bool topk_args_ok(int n_rows, int vocab, int k) {
  return n_rows >= 1 && vocab >= 1 && k >= 1 && k <= vocab && k <= 128;
}

DDT_EXPORT size_t ddt_topk_logprobs_workspace_size(int n_rows, int vocab, int k) {
  if (!topk_args_ok(n_rows, vocab, k)) return 0;
  return ddt::topk_workspace_bytes(n_rows, vocab, k);
}

DDT_EXPORT int ddt_topk_logprobs(const float* logits, int64_t ld_logits, int n_rows, int vocab,
                                 int k, float inv_temperature, int32_t* topk_ids,
                                 float* topk_logp, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!topk_args_ok(n_rows, vocab, k) || ld_logits < vocab) return DDT_EINVAL;
  if (logits == nullptr || topk_ids == nullptr || topk_logp == nullptr) return DDT_EINVAL;
  if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return DDT_EINVAL;
  if (!ddt::topk_supported(n_rows, vocab, k)) return DDT_EUNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < ddt::topk_workspace_bytes(n_rows, vocab, k))
    return DDT_EWORKSPACE;
  return launch_status(ddt::launch_topk(logits, ld_logits, n_rows, vocab, k, inv_temperature,
                                        topk_ids, topk_logp, lse, workspace,
                                        static_cast<hipStream_t>(stream)));
}

DDT_EXPORT int ddt_topk_logprobs_noalloc(const float* logits, int64_t ld_logits, int n_rows,
                                         int vocab, int k, float inv_temperature,
                                         int32_t* topk_ids, float* topk_logp, float* lse,
                                         void* stream) {
  if (!topk_args_ok(n_rows, vocab, k) || ld_logits < vocab) return DDT_EINVAL;
  if (logits == nullptr || topk_ids == nullptr || topk_logp == nullptr) return DDT_EINVAL;
  if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return DDT_EINVAL;
  if (!ddt::topk_supported(n_rows, vocab, k)) return DDT_EUNSUPPORTED;
  if (ddt::topk_workspace_bytes(n_rows, vocab, k) > DDT_TOPK_NOALLOC_SCRATCH_BYTES)
    return DDT_EWORKSPACE;
  void* scratch = nullptr;
  if (ddt::topk_noalloc_scratch(&scratch) != hipSuccess) return DDT_ELAUNCH;
  return launch_status(ddt::launch_topk(logits, ld_logits, n_rows, vocab, k, inv_temperature,
                                        topk_ids, topk_logp, lse, scratch,
                                        static_cast<hipStream_t>(stream)));
}

// ---- fused LM head + log-softmax / top-K ------------------------------------
static bool lmhead_args_ok(int n_rows, int hidden, int vocab, int k) {
  return n_rows >= 1 && hidden >= 1 && vocab >= 1 && k >= 1 && k <= vocab;
}
static bool lmhead_supported(int n_rows, int hidden, int vocab, int k) {
  const long nc = ddt::lmhead_chunks(vocab);
  return hidden % 256 == 0 && hidden <= 4096 && k <= ddt::kLmMaxK &&
         nc <= ddt::kTopkMergeMaxLists && nc * k <= ddt::kTopkMergeMaxKeys &&
         (n_rows + 15) / 16 <= 65535;
}

DDT_EXPORT size_t ddt_lmhead_topk_workspace_size(int n_rows, int hidden, int vocab, int k) {
  if (!lmhead_args_ok(n_rows, hidden, vocab, k) || !lmhead_supported(n_rows, hidden, vocab, k))
    return 0;
  return ddt::lmhead_workspace_bytes(n_rows, vocab, k);
}

DDT_EXPORT int ddt_lmhead_topk(const void* hidden_states, const void* weight, int n_rows,
                               int hidden, int vocab, int k, float inv_temperature,
                               int32_t* topk_ids, float* topk_logp, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!lmhead_args_ok(n_rows, hidden, vocab, k)) return DDT_EINVAL;
  if (hidden_states == nullptr || weight == nullptr || topk_ids == nullptr ||
      topk_logp == nullptr)
    return DDT_EINVAL;
  if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return DDT_EINVAL;
  if (!aligned16(hidden_states) || !aligned16(weight)) return DDT_EINVAL;
  if (!lmhead_supported(n_rows, hidden, vocab, k)) return DDT_EUNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < ddt::lmhead_workspace_bytes(n_rows, vocab, k))
    return DDT_EWORKSPACE;
  return launch_status(ddt::launch_lmhead_topk(hidden_states, weight, n_rows, hidden, vocab, k,
                                               inv_temperature, topk_ids, topk_logp, lse,
                                               workspace, static_cast<hipStream_t>(stream)));
}

// ---- tree positions + RoPE + K/V scatter ------------------------------------
DDT_EXPORT int ddt_tree_rope_kv(const int32_t* node_depth, const int32_t* n_nodes, int batch,
                                int n_max, const int32_t* prefix_len, const int64_t* kv_base,
                                void* q, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, int hq, int hkv, int head_dim, float rope_base,
                                int32_t* positions, void* stream) {
  if (batch < 1 || n_max < 1 || hq < 1 || hkv < 1) return DDT_EINVAL;
  if (node_depth == nullptr || n_nodes == nullptr || prefix_len == nullptr ||
      kv_base == nullptr || q == nullptr || k_new == nullptr || v_new == nullptr ||
      k_cache == nullptr || v_cache == nullptr)
    return DDT_EINVAL;
  if (!(rope_base > 1.f) || !isfinite(rope_base)) return DDT_EINVAL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return DDT_EINVAL;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return DDT_EUNSUPPORTED;
  if (batch > 65535) return DDT_EUNSUPPORTED;
  return launch_status(ddt::launch_tree_rope_kv(node_depth, n_nodes, batch, n_max, prefix_len,
                                                kv_base, q, k_new, v_new, k_cache, v_cache, hq,
                                                hkv, head_dim, rope_base, positions,
                                                static_cast<hipStream_t>(stream)));
}

// ---- target argmax --------------------------------------------------------
DDT_EXPORT size_t ddt_argmax_workspace_size(int n_rows, int vocab) {
  if (n_rows < 1 || vocab < 1) return 0;
  return ddt::argmax_workspace_bytes(n_rows, vocab);
}

DDT_EXPORT int ddt_argmax(const float* logits, int64_t ld_logits, int n_rows, int vocab,
                          int32_t* out_ids, float* out_max, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (n_rows < 1 || vocab < 1 || ld_logits < vocab) return DDT_EINVAL;
  if (logits == nullptr || out_ids == nullptr) return DDT_EINVAL;
  if (n_rows > ddt::kArgmaxMaxRows) return DDT_EUNSUPPORTED;
  const size_t need = ddt::argmax_workspace_bytes(n_rows, vocab);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return DDT_EWORKSPACE;
  return launch_status(ddt::launch_argmax(logits, ld_logits, n_rows, vocab, out_ids, out_max,
                                          workspace, static_cast<hipStream_t>(stream)));
}

// ---- stage 2 ---------------------------------------------------------------
static bool tree_args_ok(int batch, int L, int k, int k_tree, int budget) {
  return batch >= 1 && L >= 1 && L <= 32 && k >= 1 && k_tree >= 1 && k_tree <= k &&
         k_tree <= 128 && budget >= 0 && budget <= 2047;
}

static constexpr size_t kMaxLds = 160 * 1024;

DDT_EXPORT size_t ddt_build_tree_workspace_size(int batch, int L, int k, int budget) {
  (void)batch;
  (void)L;
  (void)k;
  (void)budget;
  return 0;
}

DDT_EXPORT int ddt_build_tree(const float* topk_logp, const int32_t* topk_ids,
                              const int32_t* root_token, int batch, int L, int k, int k_tree,
                              int budget, int32_t* n_nodes, int32_t* node_token,
                              int32_t* node_parent, int32_t* node_depth, float* node_score,
                              uint64_t* anc_mask, void* workspace, size_t workspace_bytes,
                              void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!tree_args_ok(batch, L, k, k_tree, budget)) return DDT_EINVAL;
  if (topk_logp == nullptr || topk_ids == nullptr || root_token == nullptr ||
      n_nodes == nullptr || node_token == nullptr || node_parent == nullptr ||
      node_depth == nullptr || anc_mask == nullptr)
    return DDT_EINVAL;
  if (ddt::tree_smem_bytes(L, k_tree, budget) > kMaxLds) return DDT_EUNSUPPORTED;
  return launch_status(ddt::launch_tree(topk_logp, topk_ids, root_token, batch, L, k, k_tree,
                                        budget, n_nodes, node_token, node_parent, node_depth,
                                        node_score, anc_mask,
                                        static_cast<hipStream_t>(stream)));
}

// ---- stage 3 ---------------------------------------------------------------
static int attn_desc_check(const ddt_attn_desc* d, bool with_mask) {
  if (d == nullptr) return DDT_EINVAL;
  if (d->batch < 1 || d->hq < 1 || d->hkv < 1 || d->hq % d->hkv != 0 || d->n_q_max < 1 ||
      d->max_kv_len < 1 || d->max_kv_len > (1 << 22))
    return DDT_EINVAL;
  if (with_mask && d->mask_words < (d->n_q_max + 63) / 64) return DDT_EINVAL;
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128) return DDT_EUNSUPPORTED;
  if (!isfinite(d->scale)) return DDT_EINVAL;
  return DDT_OK;
}

DDT_EXPORT size_t ddt_masked_attention_workspace_size(const ddt_attn_desc* desc) {
  if (attn_desc_check(desc, false) != DDT_OK) return 0;
  return ddt::attn_workspace_bytes(desc->batch, desc->hq, desc->hkv, desc->head_dim,
                                   desc->n_q_max, desc->max_kv_len);
}

DDT_EXPORT int ddt_masked_attention(const ddt_attn_desc* desc, const void* q, const void* k_cache,
                                    const void* v_cache, const int64_t* kv_base,
                                    const int32_t* prefix_len, const int32_t* n_q,
                                    const uint64_t* own_mask, void* out, float* lse_out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  const int st = attn_desc_check(desc, own_mask != nullptr);
  if (st != DDT_OK) return st;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || kv_base == nullptr ||
      prefix_len == nullptr || n_q == nullptr || out == nullptr)
    return DDT_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return DDT_EINVAL;
  const size_t need = ddt::attn_workspace_bytes(desc->batch, desc->hq, desc->hkv,
                                                desc->head_dim, desc->n_q_max, desc->max_kv_len);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return DDT_EWORKSPACE;
  const float scale = desc->scale > 0.f ? desc->scale : 1.0f / sqrtf((float)desc->head_dim);
  return launch_status(ddt::launch_attention(
      desc->batch, desc->hq, desc->hkv, desc->head_dim, desc->n_q_max, desc->mask_words,
      desc->max_kv_len, scale, q, k_cache, v_cache, kv_base, prefix_len, n_q, own_mask, 0, out,
      lse_out, workspace, static_cast<hipStream_t>(stream)));
}

DDT_EXPORT int ddt_packed_block_attention(const ddt_attn_desc* desc, int block_len, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const int64_t* kv_base, const int32_t* prefix_len,
                                          const int32_t* n_q, void* out, float* lse_out,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  const int st = attn_desc_check(desc, false);
  if (st != DDT_OK) return st;
  if (block_len < 1) return DDT_EINVAL;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || kv_base == nullptr ||
      prefix_len == nullptr || n_q == nullptr || out == nullptr)
    return DDT_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return DDT_EINVAL;
  const size_t need = ddt::attn_workspace_bytes(desc->batch, desc->hq, desc->hkv,
                                                desc->head_dim, desc->n_q_max, desc->max_kv_len);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return DDT_EWORKSPACE;
  const float scale = desc->scale > 0.f ? desc->scale : 1.0f / sqrtf((float)desc->head_dim);
  return launch_status(ddt::launch_attention(
      desc->batch, desc->hq, desc->hkv, desc->head_dim, desc->n_q_max, 0, desc->max_kv_len, scale,
      q, k_cache, v_cache, kv_base, prefix_len, n_q, nullptr, block_len, out, lse_out, workspace,
      static_cast<hipStream_t>(stream)));
}

// ---- stage 4 ---------------------------------------------------------------
DDT_EXPORT int ddt_accept_compact(const int32_t* node_token, const int32_t* node_parent,
                                  const int32_t* n_nodes, int n_max,
                                  const int32_t* target_argmax, int batch, int L, void* k_cache,
                                  void* v_cache, const int64_t* kv_base,
                                  const int32_t* prefix_len, int n_layers,
                                  int64_t layer_stride_elems, int hkv, int head_dim,
                                  int32_t* accept_len, int32_t* accepted_nodes,
                                  int32_t* bonus_token, int32_t* new_len, void* stream) {
  if (batch < 1 || n_max < 1 || L < 1 || n_layers < 0 || hkv < 1 || head_dim < 1 ||
      (hkv * head_dim) % 8 != 0)
    return DDT_EINVAL;
  if (node_token == nullptr || node_parent == nullptr || n_nodes == nullptr ||
      target_argmax == nullptr || prefix_len == nullptr || accept_len == nullptr ||
      accepted_nodes == nullptr || bonus_token == nullptr || new_len == nullptr)
    return DDT_EINVAL;
  if (n_layers > 0) {
    if (k_cache == nullptr || v_cache == nullptr || kv_base == nullptr) return DDT_EINVAL;
    if (!aligned16(k_cache) || !aligned16(v_cache) || (layer_stride_elems % 8) != 0)
      return DDT_EINVAL;
  }
  if ((size_t)(n_max + L + 3) * sizeof(int) > kMaxLds) return DDT_EUNSUPPORTED;
  if (n_layers > 65535) return DDT_EUNSUPPORTED;  // layers are the grid's y dimension
  return launch_status(ddt::launch_accept(node_token, node_parent, n_nodes, n_max,
                                          target_argmax, batch, L, k_cache, v_cache, kv_base,
                                          prefix_len, n_layers, layer_stride_elems, hkv,
                                          head_dim, accept_len, accepted_nodes, bonus_token,
                                          new_len, static_cast<hipStream_t>(stream)));
}
