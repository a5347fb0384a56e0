/*
 * ddt.h -- C ABI of the DFlash + DDTree draft-and-verify kernel chain for
 * AMD Instinct MI355X (gfx950).
 *
 * One speculative decoding step runs four stages on the GPU:
 *   1. ddt_topk_logprobs     per-position log-softmax + top-K over the vocab
 *   2. ddt_build_tree        best-first top-B prefix tree, flattened, with
 *                            parent/depth arrays and an ancestor bitmask
 *   3. ddt_masked_attention  GQA attention of the query rows over a prefix KV
 *                            cache plus their own KV rows, with either the
 *                            ancestor-only tree mask (verify) or a dense own
 *                            block (drafter pass over injected context KV)
 *   4. ddt_accept_compact    greedy acceptance walk against the target's
 *                            argmax tokens + compaction of the accepted KV rows
 * and, between 3 and 4, ddt_argmax: the target's greedy token per tree slot
 * (a vocab-wide arg-max over the verify logits); ddt_lmhead_topk feeds stage
 * 1 from the drafter's hidden states through the shared LM head.
 *
 * Pages the operations come from (cited by title and section):
 *   [DDTree]  "Accelerating Speculative Decoding with Block Diffusion Draft
 *             Trees" summary (bluediary8.tistory.com/1288)
 *   [DFlash]  "DFlash: Block Diffusion for Flash Speculative Decoding"
 *             summary (honbul.tistory.com/178)
 *   [DFlash-news]  DFlash article (darkpulse.kr/?p=2484)
 *
 * Conventions shared by every call
 *   - Array arguments are DEVICE pointers unless marked "host".  The caller
 *     owns all memory; the library never allocates, frees or synchronizes.
 *   - Every call is asynchronous on the caller's stream (hipStream_t passed
 *     as void*; NULL = the null stream).
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     an error nothing is launched and outputs are untouched.
 *   - Device-side preconditions (finite logits, sorted top-K tables, cache
 *     capacity) are documented per call and not checked.
 *   - Layouts are row-major with the last dimension contiguous.  bf16 data
 *     is passed as void* and holds IEEE bfloat16 bit patterns.
 *   - No C++ exception crosses this boundary.
 */
#ifndef DDT_H
#define DDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DDT_OK 0
#define DDT_EINVAL 1        /* bad size, null required pointer, bad relation */
#define DDT_EUNSUPPORTED 2  /* head_dim or shape outside what the kernels build for */
#define DDT_EWORKSPACE 3    /* workspace pointer NULL or smaller than required */
#define DDT_ELAUNCH 4       /* the HIP runtime reported an error at launch */

#define DDT_ABI_VERSION 1

int ddt_abi_version(void);
const char* ddt_status_string(int status);

/* ------------------------------------------------------------------------
 * Stage 1: per-position log-softmax and top-K.
 *
 * [DDTree] "핵심 아이디어" (core idea): the drafter emits one distribution over
 * the vocabulary per masked block position in a single forward pass; the
 * tree builder reads them as log-probabilities.  K (candidates kept per
 * position) is a workload parameter; the pages fix none.
 *
 * For each row r (0 <= r < n_rows):
 *   x_v     = fl32(logits[r*ld_logits + v] * inv_temperature)
 *   lse[r]  = log(sum_v exp(x_v))                 (float32 result)
 *   ids     = the k tokens with the largest x, ties to the smaller id,
 *             in that order (ranking on the float32 x)
 *   logp_j  = x_{ids_j} - lse[r]                  (<= 0, non-increasing in j)
 *
 * logits     f32 [n_rows, ld_logits]  (only the first vocab columns are read)
 * topk_ids   i32 [n_rows, k]          (output)
 * topk_logp  f32 [n_rows, k]          (output)
 * lse        f32 [n_rows]             (output, may be NULL)
 * workspace  device scratch of ddt_topk_logprobs_workspace_size() bytes;
 *            contents on entry are ignored.
 * Errors: EINVAL if n_rows < 1, vocab < 1, k < 1, k > vocab, k > 128,
 *         ld_logits < vocab, a required pointer is NULL, or
 *         inv_temperature is not a positive finite number; EUNSUPPORTED if
 *         n_rows > 65535.
 * Preconditions (device): logits finite.
 * ---------------------------------------------------------------------- */
size_t ddt_topk_logprobs_workspace_size(int n_rows, int vocab, int k);
int ddt_topk_logprobs(const float* logits, int64_t ld_logits, int n_rows, int vocab,
                      int k, float inv_temperature, int32_t* topk_ids, float* topk_logp,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 1 without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same definition, arguments, outputs and errors as ddt_topk_logprobs; the
 * per-chunk partials go to a scratch array that the library holds in device
 * memory of each GPU it runs on (DDT_TOPK_NOALLOC_SCRATCH_BYTES, held until
 * the process ends).  The call allocates nothing.  Its first call on a
 * device looks up that device's scratch address (no allocation; make it
 * outside graph capture).
 * Extra error: EWORKSPACE if the shape needs more scratch than
 *   DDT_TOPK_NOALLOC_SCRATCH_BYTES (ddt_topk_logprobs_workspace_size() tells
 *   how much), ELAUNCH if the scratch address cannot be looked up.
 * Every call on one GPU uses that GPU's one scratch array: calls that
 * overlap on one GPU (concurrent streams, threads) race and must not be
 * issued; calls in one stream are ordered and safe.
 * ---------------------------------------------------------------------- */
#define DDT_TOPK_NOALLOC_SCRATCH_BYTES (8u << 20)
int ddt_topk_logprobs_noalloc(const float* logits, int64_t ld_logits, int n_rows, int vocab,
                              int k, float inv_temperature, int32_t* topk_ids,
                              float* topk_logp, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Fused LM head + log-softmax / top-K (stage 1 fed from hidden states).
 *
 * [DFlash] "임베딩과 출력 헤드는 공유한다" (embedding and output head are
 * shared): the drafter's output head is the target's frozen LM head, so the
 * per-position logits are one GEMM of the drafter's block hidden states with
 * that weight.  This call computes them on MFMA and reduces them to the
 * stage-1 outputs in the same pass: the logits never reach HBM.
 *
 * For each row r (0 <= r < n_rows):
 *   z_v   = sum_h hidden_states[r, h] * weight[v, h]   (bf16 products, fp32
 *           accumulation; the summation order is the kernel's)
 *   x_v   = fl32(z_v * inv_temperature)
 *   then exactly the ddt_topk_logprobs definition on x: lse, the k largest
 *   x (ties to the smaller id), logp = x - lse.
 *
 * hidden_states bf16 [n_rows, hidden]   weight bf16 [vocab, hidden] (row v =
 *   the output embedding of token v); both 16-byte aligned.
 * topk_ids i32 [n_rows, k], topk_logp f32 [n_rows, k], lse f32 [n_rows]
 *   (may be NULL).
 * workspace: ddt_lmhead_topk_workspace_size() bytes (chunk partials); its
 *   contents on entry are ignored.  The weight is read once per block of 16
 *   rows, so the call is meant for the drafter's few block rows.
 * Errors: EINVAL if n_rows < 1, hidden < 1, vocab < 1, k < 1, k > vocab, a
 *         required pointer is NULL or misaligned, or inv_temperature is not
 *         a positive finite number; EUNSUPPORTED if hidden is not a
 *         multiple of 256 or exceeds 4096, k > 64, or the vocabulary needs
 *         more than 256 chunks of 640 (vocab > 163840) or
 *         chunks * k > 16384; EWORKSPACE if the workspace is too small.
 * Preconditions (device): finite inputs.
 * ---------------------------------------------------------------------- */
size_t ddt_lmhead_topk_workspace_size(int n_rows, int hidden, int vocab, int k);
int ddt_lmhead_topk(const void* hidden_states, const void* weight, int n_rows, int hidden,
                    int vocab, int k, float inv_temperature, int32_t* topk_ids,
                    float* topk_logp, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ------------------------------------------------------------------------
 * Tree positions + rotary embedding + tree K/V scatter (between stages 2
 * and 3b, one layer per call).
 *
 * [DDTree] "방법론 자세히 보기" (method in detail): the flattened tree is
 * verified in one target pass, each token continuing the sequence after its
 * own ancestors.  So the token in slot i sits at position P + depth[i] (the
 * root, the bonus token, at P), not at P + i; a chain gives the ordinary
 * positions.  The pages do not name the positional encoding; this call
 * applies the rotary one in its common split-half form:
 *   theta_j = rope_base^(-2j/D), a = pos * theta_j  (j < D/2)
 *   (x_j, x_{j+D/2}) -> (x_j cos a - x_{j+D/2} sin a,
 *                        x_{j+D/2} cos a + x_j sin a)
 * evaluated in double precision and rounded to float, then to bf16 (both
 * round to nearest even).
 *
 * For request b and slot i < n_nodes[b] (P = prefix_len[b]):
 *   positions[b, i] = P + node_depth[b, i]     (-1 for slots >= n_nodes)
 *   q[b, i, h, :]   rotated in place           (every q head h < hq)
 *   k_cache[kv_base[b] + P + i, g, :] = rotate(k_new[b, i, g, :])
 *   v_cache[kv_base[b] + P + i, g, :] = v_new[b, i, g, :]
 * Slots >= n_nodes[b] are not read or written (q rows stay as they are).
 *
 * node_depth i32 [batch, n_max]; n_nodes, prefix_len i32 [batch];
 * kv_base i64 [batch]; q bf16 [batch, n_max, hq, D]; k_new, v_new bf16
 * [batch, n_max, hkv, D]; k_cache, v_cache bf16 [rows, hkv, D];
 * positions i32 [batch, n_max] or NULL.  Tensors 16-byte aligned.
 * Errors: EINVAL if batch < 1, n_max < 1, hq < 1, hkv < 1, a required
 *         pointer is NULL or misaligned, or rope_base is not a finite
 *         number > 1; EUNSUPPORTED if head_dim is not 32, 64, 128 or 256 or
 *         batch > 65535.
 * Preconditions (device): cache rows kv_base[b] + P .. + n_nodes[b] - 1
 *   exist; n_nodes[b] <= n_max.
 * ---------------------------------------------------------------------- */
int ddt_tree_rope_kv(const int32_t* node_depth, const int32_t* n_nodes, int batch, int n_max,
                     const int32_t* prefix_len, const int64_t* kv_base, void* q,
                     const void* k_new, const void* v_new, void* k_cache, void* v_cache, int hq,
                     int hkv, int head_dim, float rope_base, int32_t* positions, void* stream);

/* ------------------------------------------------------------------------
 * Target argmax: the verifier's greedy token for every tree slot.
 *
 * [DDTree] "방법론 자세히 보기" (method in detail): the target model runs once
 * over the flattened tree and the verifier compares its outputs with the
 * tree; with greedy decoding the output at a slot is the target's most
 * probable token there.  These ids are the target_argmax input of
 * ddt_accept_compact.
 *
 * For each row r (0 <= r < n_rows):
 *   out_ids[r] = the smallest v in [0, vocab) with
 *                logits[r*ld_logits + v] = max_u logits[r*ld_logits + u]
 *   out_max[r] = that maximum (a maximum of -0 is reported as +0; -0 and +0
 *                tie, and the smaller index wins)
 * No temperature: the arg-max of z/T equals that of z for T > 0 up to ties
 * created by rounding, and greedy verification uses the raw logits.
 *
 * logits    f32 [n_rows, ld_logits] (only the first vocab columns are read)
 * out_ids   i32 [n_rows]  (output)
 * out_max   f32 [n_rows]  (output, may be NULL)
 * workspace ddt_argmax_workspace_size() bytes of device scratch (chunk
 *           partials; 0 -- workspace may be NULL -- when a row fits one
 *           chunk); contents on entry are ignored.
 * Errors: EINVAL if n_rows < 1, vocab < 1, ld_logits < vocab, or logits /
 *         out_ids is NULL; EUNSUPPORTED if n_rows > 65535; EWORKSPACE if
 *         the workspace is needed and missing or too small.
 * Preconditions (device): no NaN among the logits (+-inf is allowed).
 * ---------------------------------------------------------------------- */
size_t ddt_argmax_workspace_size(int n_rows, int vocab);
int ddt_argmax(const float* logits, int64_t ld_logits, int n_rows, int vocab, int32_t* out_ids,
               float* out_max, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 2: DDTree best-first tree build, flattened.
 *
 * [DDTree] "방법론 자세히 보기" (method in detail): under the factorized
 * (position-independent) draft distribution the expected acceptance length
 * is the sum of the tree's prefix probabilities, so the optimal tree of
 * budget B holds the B most probable prefixes; a best-first max-heap finds
 * them in O(B log B).  The tree is flattened for one verify pass under an
 * ancestor-only mask ("용어 정리" / glossary).
 *
 * Per request b (rows [b*L, (b+1)*L) of the top-K tables; row d-1 serves
 * depth d):
 *   slot 0     root = root_token[b], parent -1, depth 0, score 0
 *   slots 1..  the `budget` best non-empty prefixes whose depth-d token has
 *              rank < k_tree in row d-1, score(child) = fl32(score(parent)
 *              + topk_logp[d-1][rank]), ordered by the canonical key
 *              (score desc, depth asc, parent slot asc, rank asc) -- the
 *              best-first pop order, so parents precede children
 *   n_nodes[b] 1 + number of prefixes taken (< budget+1 only when fewer
 *              than `budget` prefixes exist)
 *   anc_mask   bit j of row i (word j/64, bit j%64) set iff slot j is slot
 *              i or one of its ancestors (root included)
 *   slots >= n_nodes: token/parent/depth -1, score -inf, mask row 0.
 *
 * topk_logp  f32 [batch*L, k]   non-positive, non-increasing along k
 * topk_ids   i32 [batch*L, k]   distinct within a row
 * root_token i32 [batch]
 * outputs (n_max = budget+1, W = ceil(n_max/64)):
 *   n_nodes i32 [batch]; node_token, node_parent, node_depth i32 [batch, n_max];
 *   node_score f32 [batch, n_max] (may be NULL); anc_mask u64 [batch, n_max, W]
 * workspace: ddt_build_tree_workspace_size() bytes (currently 0; may be NULL).
 * Errors: EINVAL if batch < 1, L < 1 or L > 32, k < 1, k_tree < 1,
 *         k_tree > k, k_tree > 128, budget < 0 or budget > 2047, or a
 *         required pointer is NULL; EUNSUPPORTED if the selection buffer for
 *         (budget, k_tree) does not fit in on-chip memory.
 * ---------------------------------------------------------------------- */
size_t ddt_build_tree_workspace_size(int batch, int L, int k, int budget);
int ddt_build_tree(const float* topk_logp, const int32_t* topk_ids, const int32_t* root_token,
                   int batch, int L, int k, int k_tree, int budget, int32_t* n_nodes,
                   int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                   float* node_score, uint64_t* anc_mask, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 3: masked GQA attention.
 *
 * Verify mode (own_mask != NULL) -- [DDTree] "방법론 자세히 보기" and "용어
 * 정리": the flattened tree is checked in one target pass; each tree token
 * sees the committed prefix and, inside the tree, only its ancestor path
 * (itself included).  Drafter mode (own_mask == NULL) -- [DFlash]
 * "DFlash의 핵심 아이디어" points 2-3 and [DFlash-news] "DFlash 핵심 기술 구조":
 * target context is injected as key/value memory into the draft layers and
 * the masked block is filled jointly, so block queries see every context
 * row and every row of their own block.
 *
 * Request r owns cache rows kv_base[r] + [0, prefix_len[r]) (prefix /
 * context) and kv_base[r] + prefix_len[r] + [0, n_q[r]) (the queries' own
 * K/V, row i for query i).  Query i of request r, head h, reads KV head
 * h / (hq/hkv) and attends to
 *   every prefix row, and own row j iff (own_mask == NULL && j < n_q[r]) or
 *   bit j of own_mask[(r*n_q_max + i)*mask_words + j/64] is set.
 *   out = softmax(scale * q.K^T over the visible rows) . V
 *   lse = log(sum exp(scale * q.k)) over the visible rows (natural log)
 * Arithmetic: bf16 inputs, fp32 accumulation; out rounded to bf16 (RNE).
 *
 * q        bf16 [batch, n_q_max, hq, D]
 * k_cache, v_cache  bf16 [rows, hkv, D]
 * kv_base  i64 [batch];  prefix_len, n_q  i32 [batch] (0 <= n_q <= n_q_max)
 * own_mask u64 [batch, n_q_max, mask_words] or NULL
 * out      bf16 [batch, n_q_max, hq, D]; rows i >= n_q[r] are not written
 * lse_out  f32 [batch, n_q_max, hq] or NULL
 * desc->max_kv_len: host-known upper bound on prefix_len[r] + n_q[r]; it
 *   sizes the launch grid.  desc->scale <= 0 selects 1/sqrt(D).
 * workspace: ddt_masked_attention_workspace_size(desc) bytes (split-KV
 *   partial results); contents on entry are ignored.
 * Errors: EINVAL if batch < 1, hq < 1, hkv < 1, hq % hkv != 0, n_q_max < 1,
 *         max_kv_len < 1 or > 2^22, mask_words < ceil(n_q_max/64) with a
 *         mask, a required pointer is NULL, or q / k_cache / v_cache / out
 *         is not 16-byte aligned; EUNSUPPORTED if D is not 32, 64 or 128.
 * Preconditions (device): prefix_len[r] + n_q[r] <= desc->max_kv_len and
 *   every referenced cache row exists.
 * ---------------------------------------------------------------------- */
typedef struct {
  int batch;
  int hq;
  int hkv;
  int head_dim;
  int n_q_max;
  int mask_words;
  int max_kv_len;
  float scale;
} ddt_attn_desc;

size_t ddt_masked_attention_workspace_size(const ddt_attn_desc* desc);
int ddt_masked_attention(const ddt_attn_desc* desc, const void* q, const void* k_cache,
                         const void* v_cache, const int64_t* kv_base, const int32_t* prefix_len,
                         const int32_t* n_q, const uint64_t* own_mask, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 3, packed drafter blocks: block-diagonal own-row visibility.
 *
 * [DFlash] "여러 블록을 한 번에 학습하되, 블록끼리 새지 않게 막는다"
 * (several blocks are processed in one sequence, kept from leaking into one
 * another): the drafter's attention mask lets rows of one block see each
 * other but no row of another block.  Here the own rows of request r are
 * cut into consecutive blocks of block_len rows (the last one may be
 * shorter); query i sees every prefix (context) row and the own rows j with
 * j / block_len == i / block_len.  Everything else -- layouts, arithmetic,
 * outputs, workspace (ddt_masked_attention_workspace_size) -- is exactly
 * ddt_masked_attention in drafter mode, which block_len >= n_q reproduces.
 * Errors: those of ddt_masked_attention, plus EINVAL if block_len < 1.
 * ---------------------------------------------------------------------- */
int ddt_packed_block_attention(const ddt_attn_desc* desc, int block_len, const void* q,
                               const void* k_cache, const void* v_cache, const int64_t* kv_base,
                               const int32_t* prefix_len, const int32_t* n_q, void* out,
                               float* lse_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Stage 4: greedy acceptance walk + KV compaction.
 *
 * [DDTree] "방법론 자세히 보기": the verifier follows the tree along the
 * target's outputs, accepts the longest matching path and removes the
 * rejected branches from the KV cache.  Greedy (temperature 0) rule:
 *   cur = 0; path = [0]
 *   while a child c of cur has node_token[c] == target_argmax[cur]:
 *     append c; cur = c
 *   accept_len = |path| - 1; bonus_token = target_argmax[cur]
 *   for every layer, cache rows P + path[j] move to rows P + j
 *   (P = prefix_len[b]; all source rows are read before any is written)
 *   new_len = P + accept_len + 1
 *
 * node_token, node_parent, target_argmax  i32 [batch, n_max]; n_nodes i32 [batch]
 * k_cache, v_cache  bf16, layer l at k_cache + l*layer_stride_elems, rows of
 *   hkv*head_dim elements; request b's tree rows start at kv_base[b] + P.
 * outputs: accept_len, bonus_token, new_len i32 [batch];
 *   accepted_nodes i32 [batch, L+1] (path, then -1)
 * Rows >= new_len of the request are unspecified afterwards.  Accepted
 * paths of any length up to L are compacted: more than 1024 path rows are
 * moved in several register rounds, in increasing path order.
 * Errors: EINVAL if batch < 1, n_max < 1, L < 1, n_layers < 0, hkv < 1,
 *         head_dim < 1, hkv*head_dim not a multiple of 8, or a required
 *         pointer is NULL; EUNSUPPORTED if n_layers > 65535 or the slot
 *         table (n_max + L + 3 words) exceeds 160 KiB of on-chip memory.
 * Preconditions (device): a tree as ddt_build_tree writes it (parents
 *   precede children, sibling tokens distinct, depth <= L).
 * ---------------------------------------------------------------------- */
int ddt_accept_compact(const int32_t* node_token, const int32_t* node_parent,
                       const int32_t* n_nodes, int n_max, const int32_t* target_argmax,
                       int batch, int L, void* k_cache, void* v_cache, const int64_t* kv_base,
                       const int32_t* prefix_len, int n_layers, int64_t layer_stride_elems,
                       int hkv, int head_dim, int32_t* accept_len, int32_t* accepted_nodes,
                       int32_t* bonus_token, int32_t* new_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DDT_H */
