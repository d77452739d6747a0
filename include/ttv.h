/*
 * ttv.h -- token-tree verification hot path on AMD Instinct MI355X (gfx950).
 *
 * One speculative verify round over a batch of draft trees:
 *   draft_tree_expand,   grow each round's tree from the drafter's
 *   draft_tree_select    confidence (expand by top-k, rerank by path score)
 *   tree_build_mask      ancestor bitsets from a per-round parent[] topology
 *   tree_verify_attention tree-masked GQA attention over the KV prefix plus
 *                        each node's ancestors
 *   vocab_argmax         per-node argmax over the target's vocabulary logits
 *   vocab_sample         per-node draw from the nucleus-filtered distribution
 *                        (the sampled form of the target's selection)
 *   lm_head_argmax       the argmax fused with the LM-head projection, the
 *                        logits never written (lm_head_q4_argmax: 4-bit head)
 *   tree_accept_walk     descend the one child matching the target's argmax
 *   kv_gather_positions  compact the accepted path's K/V (and int8 scales)
 *                        along the sequence axis
 * and the sliding-window layers' variants: sliding_mask_from_caller (caller
 * mask intersected with the window band), tree_verify_attention_window (the
 * attention under that band) and kv_gather_within_tail (the rollback confined
 * to the verify block, refusing a wrapped rotating cache).
 *
 * Sources are cited by page title and section:
 *   [I1204]  mlxcel issue #1204 "perf(speculative): draft a tree instead of a
 *            chain, so an MTP round emits more than 2.33 tokens"
 *   [PR1212] mlxcel PR #1212 "feat(speculative): draft and verify a token
 *            tree, behind a flag, default off" (its commit messages)
 *   [I1185]  mlxcel issue #1185 "perf(speculative): cut the MTP drafter's
 *            per-step cost" (its "Proposed work" phases)
 *   [S728]   splash issue #728 "Experiment: qualify shared-prefix tree
 *            verification and conservative admission"
 *
 * Conventions for every call
 *  - Pointers marked (device) are device memory; (host) are host memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *    stream). The library never synchronises, never allocates and holds no
 *    state apart from a thread-local error string (and, for
 *    tree_verify_attention_static, a static device scratch array and its
 *    per-device address). The caller owns every buffer, including
 *    workspaces sized by the *_ws queries.
 *  - Return value: TTV_OK, or an error code with a reason in ttv_last_error().
 *    TTV_ERR_INVALID and TTV_ERR_UNSUPPORTED are decided on the host before
 *    anything is launched, so nothing has been written when they return.
 *  - Kernel-side validation (of data only the device sees) reports through a
 *    caller-provided `dev_status` int32 (device): kernels only ever store a
 *    nonzero TTV_DEV_* code into it, so the caller zeroes it beforehand and
 *    reads it at its next synchronisation point.
 *  - Limits: B <= TTV_MAX_BATCH sequences, T_b <= 64 nodes per tree.
 */
#ifndef TTV_H
#define TTV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTV_MAX_BATCH 128
#define TTV_MAX_NODES 64

typedef enum ttv_status {
  TTV_OK = 0,
  TTV_ERR_INVALID = 1,     /* malformed shapes/metadata; nothing launched */
  TTV_ERR_UNSUPPORTED = 2, /* a named refusal: the caller must decline the tree round */
  TTV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_ws query */
  TTV_ERR_HIP = 4          /* a HIP launch error */
} ttv_status;

/* Device-side status codes (stored into dev_status). */
#define TTV_DEV_OK 0
#define TTV_DEV_BAD_PARENT 1    /* parent[0] != -1 or parent[i] not in [0, i) */
#define TTV_DEV_BAD_SELECTION 2 /* selection not strictly increasing / out of range / too long */
#define TTV_DEV_BAD_LOGITS 3    /* a drafter logit row holds a NaN or an infinity */
#define TTV_DEV_DRAFT_STATE 4   /* a draft candidate table cannot take the call (see draft_tree_expand) */

typedef enum ttv_dtype {
  TTV_F32 = 0,  /* float32 */
  TTV_BF16 = 1, /* bfloat16 */
  TTV_I8 = 2    /* int8 codes with fp16 per-token scale sidecars (KV only) */
} ttv_dtype;

/*
 * A batch of draft trees. Sequence b owns block nodes
 * [node_off[b], node_off[b+1]) of every node-indexed array, listed in
 * topological order (parent precedes child; node 0 of each tree is its root,
 * the last committed token) [I1204] "Increment 1". hist_len[b] is the live
 * cache length before the verify block (P_b): the block's K/V rows are
 * already appended at [P_b, P_b + T_b) in node order [PR1212] rollback-to-path
 * commit. The host and device copies must hold the same values.
 */
typedef struct ttv_batch {
  int32_t B;
  const int32_t* node_off_h; /* (host)   [B+1], node_off[0] == 0, non-decreasing */
  const int32_t* hist_len_h; /* (host)   [B] */
  const int32_t* node_off_d; /* (device) [B+1] */
  const int32_t* hist_len_d; /* (device) [B] */
} ttv_batch;

/*
 * One layer's KV cache: k and v are [B][Hkv][cap][D] contiguous, the sequence
 * axis third ([PR1212] commit widening the gather: every per-token buffer sits
 * on axis 2). For TTV_I8, k_scale and v_scale are fp16 bit patterns
 * [B][Hkv][cap], one scale per (token, KV head): value = code * scale.
 */
typedef struct ttv_kv_layer {
  void* k;            /* (device) */
  void* v;            /* (device) */
  uint16_t* k_scale;  /* (device) fp16, required iff dtype == TTV_I8, else NULL */
  uint16_t* v_scale;  /* (device) fp16, required iff dtype == TTV_I8, else NULL */
  int32_t dtype;      /* ttv_dtype */
  int32_t Hkv;
  int32_t D;
  int32_t cap;        /* allocated rows per (b, head) */
} ttv_kv_layer;

/*
 * Before step 1 -- growing the draft tree from drafter confidence [I1204]
 * "What this needs" (where the branches go: EAGLE-2 branches by drafter
 * confidence, which needs the drafter's logits past their argmax); [PR1212]
 * Drafter::draft_tree commit (a non-branching drafter gives a linear tree;
 * the runner-up at an uncertain step is the alternative worth verifying);
 * [S728] "What it does" (the chain plus alternatives from a top-k selector).
 * Reading: EAGLE-2's expand-then-rerank. A candidate's score is its float64
 * path log-probability, the sum of the drafter's log-softmax along the path.
 *
 * Per sequence b the caller owns a candidate table of cand_cap entries
 * (cand_cap <= 4096) and a frontier of top_k slots:
 *   cand_token, cand_parent (device) int32 [B][cand_cap]; parent is a
 *                       candidate index of the same sequence, -1 = the root
 *   cand_score  (device) float64 [B][cand_cap]
 *   cand_count  (device) int32 [B]       candidates in the table
 *   frontier    (device) int32 [B][top_k] candidate indices, best first
 *
 * draft_tree_expand adds one depth to every sequence's table. depth == 1
 * starts afresh (the count is reset, the frontier is the root alone, one row
 * per sequence); depth > 1 expands the frontier the previous call left.
 *   logits (device) fp32, row b * F + f at logits + row * row_stride is the
 *          drafter's row for frontier slot f of sequence b; F = 1 at depth 1
 *          and top_k after. Rows must be finite.
 * Each row's top_k tokens (by fp32 logit, ties to the lower token) are
 * appended, row by row and best first, as children of that frontier node,
 * scored parent score + logit - log(sum(exp(row))); the new frontier is the
 * top_k of those F * top_k candidates by score (ties to the lower index).
 * Limits (TTV_ERR_INVALID): 1 <= B <= TTV_MAX_BATCH, 1 <= top_k <= 16,
 * top_k <= vocab <= 2^31 - 1, row_stride >= vocab, top_k <= cand_cap <= 4096,
 * ceil(vocab / 2048) * top_k <= 65536. ws: >= draft_tree_expand_ws(B * F,
 * vocab, top_k) bytes, contents irrelevant. Device checks: a row with a NaN
 * or an infinity stores TTV_DEV_BAD_LOGITS; a table without room for the
 * depth (count + F * top_k > cand_cap) or without a frontier stores
 * TTV_DEV_DRAFT_STATE. Either leaves that sequence's table untouched.
 *
 * draft_tree_select writes each sequence's tree of n_nodes (<= 64) nodes at
 * parent/token[b * n_nodes ...] (so node_off[b] = b * n_nodes for the calls
 * below): node 0 is root_token[b] with parent -1; nodes 1.. are the
 * n_nodes - 1 best candidates of the table by score (ties to the lower
 * index), labelled in that order, which is topological. node_score (device,
 * nullable) float64 [B * n_nodes] gets the scores (0 for the root). A table
 * with fewer than n_nodes - 1 candidates, or one whose chosen set is not
 * closed under parents, stores TTV_DEV_DRAFT_STATE and writes nothing for
 * that sequence.
 */
size_t draft_tree_expand_ws(int32_t n_rows, int64_t vocab, int32_t top_k);
ttv_status draft_tree_expand(int32_t B, int32_t depth, int32_t top_k, const float* logits, int64_t vocab,
                             int64_t row_stride, int32_t* cand_token, int32_t* cand_parent, double* cand_score,
                             int32_t* cand_count, int32_t cand_cap, int32_t* frontier, int32_t* dev_status, void* ws,
                             size_t ws_bytes, void* stream);
ttv_status draft_tree_select(int32_t B, int32_t n_nodes, const int32_t* root_token, const int32_t* cand_token,
                             const int32_t* cand_parent, const double* cand_score, const int32_t* cand_count,
                             int32_t cand_cap, int32_t* parent, int32_t* token, double* node_score,
                             int32_t* dev_status, void* stream);

/*
 * Step 1 -- ancestor mask [I1204] "What this needs" (1), "Increment 3";
 * [PR1212] history-mask commit.
 * For every node i: anc[i] bit j = 1 iff block node j is i or an ancestor of
 * i; depth[i] = number of proper ancestors. Row i of the pages' additive mask
 * [T, P+T] is open (0) on all P history columns and on block column j exactly
 * when anc[i] bit j is set; the mask is rebuilt every round because the
 * topology changes.
 *   parent  (device) int32 [sum T_b], tree-local labels, parent[root] = -1
 *   anc     (device) uint64 [sum T_b]   out
 *   depth   (device) int32 [sum T_b]    out (may be NULL)
 * A tree with an invalid parent[] stores TTV_DEV_BAD_PARENT and writes no
 * anc/depth entry of that tree. Empty trees (T_b = 0) are allowed.
 */
ttv_status tree_build_mask(const ttv_batch* batch, const int32_t* parent, uint64_t* anc,
                           int32_t* depth, int32_t* dev_status, void* stream);

/*
 * Interop/test form of step 1: expand sequence b's bitsets into the pages'
 * dense additive mask out[T_b][P_b + T_b] (float32, row-major, device):
 * 0 where open, `masked` (the pages use -1e9, [PR1212] Gemma 4 tree-verify
 * commit) where blocked.
 */
ttv_status tree_mask_expand_additive(const ttv_batch* batch, int32_t b, const uint64_t* anc,
                                     float masked, float* out, void* stream);

/*
 * Sliding-window layers' form of step 1 [PR1212] the commit intersecting the
 * caller mask with the sliding band and the commit stating its properties.
 * Query row q of caller[T][S] (float32, row-major, device) sits at cache
 * position offset + q; the band keeps column c iff
 * offset + q - window < c <= offset + q. Past the window (offset + T > window)
 *   out[q][c] = min(caller[q][c], band ? 0 : masked)   (a NaN propagates)
 * and below it (offset + T <= window) out is caller, untouched, as the pages'
 * guard leaves it. Properties: an all-open caller past the window gives the
 * band; applying the call to its own output changes nothing.
 *   caller (device) float32 [T][S]; out (device) float32 [T][S], may be caller
 *          itself (in place) but must not overlap it otherwise.
 * Requires window >= 1, T <= 65535, offset >= 0.
 */
ttv_status sliding_mask_from_caller(const float* caller, int32_t T, int32_t S, int32_t offset, int32_t window,
                                    float masked, float* out, void* stream);

/*
 * Step 2 -- tree-masked GQA verify attention [I1204] "Redirection" (flatten the
 * nodes into one sequence; the tree mask hides siblings); [PR1212] history-mask
 * commit. For node i of sequence b and query head h (KV head g = h / (Hq/Hkv)):
 *   out[i][h] = sum_j softmax_j(scale * q[i][h] . k[b][g][j]) * v[b][g][j]
 * over j in [0, P_b) and j = P_b + a for every a with anc[i] bit a set.
 *   q       (device) [sum T_b][Hq][D], q_dtype TTV_F32 or TTV_BF16
 *   layer   (host)   descriptor; dtype TTV_F32, TTV_BF16 or TTV_I8
 *   anc     (device) uint64 [sum T_b] from tree_build_mask, or NULL for the
 *                    causal (linear) block mask: node i sees block rows 0..i.
 *                    A linear tree's anc gives bit-identical output to NULL.
 *   out     (device) float32 [sum T_b][Hq][D]
 *   ws      (device) >= tree_verify_attention_ws(...) bytes: the (m, l, o)
 *                    partials of units whose keys are split across
 *                    workgroups, merged by a second kernel the call enqueues.
 *                    Any contents on entry (every byte read is written first).
 * Supported: D in {64, 128}; F32 q requires F32 KV and vice versa (fp32 VALU
 * path); BF16 q with BF16 or I8 KV (MFMA path when D == 128 and cap >= 32,
 * otherwise VALU). The MFMA path forms P.V in fp16, so
 * BF16 V entries must lie within fp16 range (|v| <= 65504). With BF16 KV the
 * scores take Q as bf16. With I8 KV the scores take Q as fp16: the rows of
 * one KV head (T_b * Hq/Hkv of them, in chunks of at most 80) are multiplied
 * by one power of two that brings the chunk's largest |q| into
 * [2^14, 2^15) -- exact for every bf16 entry within a factor 2^28 of that
 * largest -- and the score scale takes the factor back out. The codes then
 * enter the matrix cores as c + 1152 with the score accumulators starting at
 * -1152 * sum_d q_d while every row of the chunk has
 * sum_d |q_d| * softmax_scale * log2(e) <= 128; past that they are converted
 * to c exactly and the accumulators start at zero. Requires Hq % Hkv == 0,
 * cap >= P_b + T_b; cache rows (and scales) past P_b + T_b are never part of
 * the result and may hold anything, non-finite values included (tested).
 * Accuracy against float64: max-abs error below 2e-3 (bf16 / int8 KV) and
 * 1e-5 (fp32) on N(0,1) keys and values with queries
 * N(0, s^2), s from 1e-6 to 300 (tested). The probabilities P and, for int8
 * KV, P' = P * v_scale are fp16, so in general the error of an output row
 * scales with sum_j p_j |v_j|: with int8 per-token k- and v-scales that
 * spread over a factor up to 2^12 within a head it stays below 2e-3 of that
 * row's largest element (tested at 2^4, 2^8, 2^12; measured ~6e-4); at
 * 2^16 it reached 4e-3 (P' overflows then, and the rows lowered to bring it
 * back into range lose fp16 precision). bf16 keys and values whose per-token
 * magnitudes spread over a factor up to 2^10 stay within the same bound
 * (tested at 2^6 and 2^10; measured ~1e-3).
 * Concurrent calls on one GPU must not share a workspace.
 */
size_t tree_verify_attention_ws(const ttv_batch* batch, int32_t Hq, const ttv_kv_layer* layer,
                                int32_t q_dtype);
ttv_status tree_verify_attention(const ttv_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                                 const ttv_kv_layer* layer, const uint64_t* anc, float softmax_scale,
                                 float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * tree_verify_attention without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and kernels, with
 * the partials kept in a static device scratch array of the library, 32 MiB
 * per device (TTV_STATIC_SCRATCH_BYTES), that every device running the
 * library holds until the process ends. Its address is looked up once per
 * device on the first call there. A call whose tree_verify_attention_ws size
 * exceeds the scratch returns TTV_ERR_UNSUPPORTED before anything is launched.
 * The call allocates nothing. Every call on one device uses that device's one
 * scratch array, which keeps the last call's contents (nothing in it needs to
 * start at zero): calls that overlap on one device, on any streams, race and
 * must be ordered by the caller. Arguments as tree_verify_attention.
 */
#define TTV_STATIC_SCRATCH_BYTES (32u << 20)
ttv_status tree_verify_attention_static(const ttv_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                                        const ttv_kv_layer* layer, const uint64_t* anc, float softmax_scale,
                                        float* out, void* stream);

/*
 * Sliding-window layers' form of step 2 [PR1212] the commit intersecting the
 * caller mask with the sliding band: as tree_verify_attention, with node i of
 * sequence b (cache row P_b + i) keeping only keys j > P_b + i - window, i.e.
 * the key set of the tree mask intersected with the band that
 * sliding_mask_from_caller applies. History keys below P_b - window + 1 are
 * not read at all, so the cost follows the window rather than the context.
 * Every row keeps its own key, so no row is empty. window >= 1 (a window of
 * at least P_b + T_b for every b gives the same key sets as
 * tree_verify_attention). Arguments, layouts, limits and accuracy as there;
 * ws >= tree_verify_attention_window_ws(..., window) bytes. The band runs on
 * the matrix cores (the same kernels as tree_verify_attention) when window
 * >= 64 and, for every sequence whose first in-band history keys are hidden
 * from some of its nodes, the in-band history holds at least one whole
 * 32-key tile beyond the tiles of those keys; otherwise, and for f32 queries,
 * on the VALU path.
 */
size_t tree_verify_attention_window_ws(const ttv_batch* batch, int32_t Hq, const ttv_kv_layer* layer,
                                       int32_t q_dtype, int32_t window);
ttv_status tree_verify_attention_window(const ttv_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                                        const ttv_kv_layer* layer, const uint64_t* anc, float softmax_scale,
                                        int32_t window, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 3 -- per-node argmax [I1204] "Increment 1" (the target emits one argmax
 * per position); [S728] "Results" (raw F32 argmax).
 *   logits  (device) float32, row r at logits + r * row_stride, vocab entries
 *   out_idx (device) int32 [n_rows]: the lowest index of the row maximum.
 * -0.0 and +0.0 compare equal; a NaN outranks every number and the first NaN
 * wins. ws: >= vocab_argmax_ws(n_rows, vocab) bytes (may be 0).
 */
size_t vocab_argmax_ws(int64_t n_rows, int64_t vocab);
ttv_status vocab_argmax(const float* logits, int64_t n_rows, int64_t vocab, int64_t row_stride,
                        int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 3, sampled -- [S728] "Historical issue and default question", "What it
 * does": for sampled requests every node draws from the target's
 * nucleus-filtered distribution with its own uniform, so the committed tokens
 * are distributed as a chain verify's; "Results": temperature 1, top-p 0.95,
 * top-k 20. Per row r:
 *   1. the top_k largest logits (ties to the lower index, as vocab_argmax);
 *   2. p_i proportional to exp(logit_i / temperature) over those, in float64,
 *      summed in descending order; C_i their cumulative fractions;
 *   3. i* = the first i with C_i >= top_p;
 *   4. out_idx[r] = the index of the first i <= i* with C_i > u * C_{i*},
 *      u = uniforms[r * uniform_stride] (i* when none does).
 * A row whose top logit is NaN (NaN outranks every number), +inf, or -inf
 * selects that logit. top_k = 1, or top_p at most the top token's mass, gives
 * vocab_argmax's answer. Feed out_idx to tree_accept_walk as its target.
 *   logits   (device) float32, row r at logits + r * row_stride
 *   uniforms (device) float32, u in [0, 1); uniform_stride >= 0 (0: one
 *            uniform for every row)
 *   out_idx  (device) int32 [n_rows]
 * Limits (TTV_ERR_INVALID): 1 <= top_k <= 64, temperature positive and
 * finite, 0 <= top_p <= 1, n_rows <= 65535, ceil(vocab / 4096) * min(top_k,
 * vocab) <= 65536. ws: >= vocab_sample_ws(n_rows, vocab, top_k) bytes,
 * contents on entry are irrelevant.
 */
size_t vocab_sample_ws(int64_t n_rows, int64_t vocab, int32_t top_k);
ttv_status vocab_sample(const float* logits, int64_t n_rows, int64_t vocab, int64_t row_stride,
                        const float* uniforms, int64_t uniform_stride, float temperature, int32_t top_k,
                        float top_p, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 3, fused with the LM head -- [I1185] mlxcel issue #1185 "Proposed
 * work", Phase 2a: at temperature 0 the vocabulary-wide logits exist only for
 * their argmax, so the projection and the argmax are fused and the logits are
 * never written. out_idx[n] = the lowest v maximising
 * sum_i hidden[n][i] * weight[v][i] (fp32 accumulation of exact bf16
 * products; -0.0 == +0.0; a NaN outranks every number).
 *   hidden (device) bf16 [n_rows][hidden_stride], the nodes' final hidden states
 *   weight (device) bf16 [vocab][weight_stride], one vocabulary row per H-vector
 *   out_idx (device) int32 [n_rows]
 * Limits (TTV_ERR_INVALID): 0 <= n_rows <= 2^24, 1 <= vocab <= 2^31 - 1,
 * hidden_dim a positive multiple of 64 (<= 2^20), strides >= hidden_dim and
 * multiples of 8, hidden and weight 16-byte aligned. ws: >=
 * lm_head_argmax_ws(n_rows, vocab) bytes, contents irrelevant. The weight is
 * read once per 128 nodes.
 */
size_t lm_head_argmax_ws(int64_t n_rows, int64_t vocab);
ttv_status lm_head_argmax(const uint16_t* hidden, int64_t n_rows, int64_t hidden_stride, const uint16_t* weight,
                          int64_t vocab, int64_t hidden_dim, int64_t weight_stride, int32_t* out_idx, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * The same fused argmax over a 4-bit head, the form the pages' engine holds
 * the head in ([I1185] "The cost model": 248,320 x 5,120 codes plus a scale
 * and a bias per group, 715.2 MB; the "Phase 3 done" comment: affine
 * group-64 4-bit; "Proposed work" Phase 2a and its verdict: a quantised
 * matmul with argmax). weight[v][i] = scale[g][v] * code[v][i] + bias[g][v],
 * g = i / 64, code in 0..15.
 *   hidden     (device) bf16 [n_rows][hidden_stride]
 *   wq         (device) uint32 [vocab][hidden_dim / 8], 8-byte aligned: hidden
 *                       element i of row v in bits 4 (i mod 8) of word i / 8
 *   scale_bias (device) bf16 [hidden_dim / 64][vocab][2] (scale, bias),
 *                       group-major, 16-byte aligned
 *   out_idx    (device) int32 [n_rows]: lowest index of the largest logit
 * Each group's products accumulate in fp32 from exact bf16 codes and are
 * folded in as scale * partial; the bias term, sum over groups of bias times
 * the group's sum of hidden values, is a second matrix-core product, 32
 * groups at a time: the group sums (fp32, in order) enter it as three exact
 * bf16 terms, whose products accumulate in fp32 onto the same logits.
 * Limits (TTV_ERR_INVALID): 0 <= n_rows <= 2^24, vocab a multiple of 4,
 * hidden_dim a positive multiple of 64 (<= 2^20), hidden_stride >= hidden_dim
 * and a multiple of 8. ws: >= lm_head_q4_argmax_ws(n_rows, vocab, hidden_dim)
 * bytes, contents irrelevant (0 for hidden_dim < 64). The codes are read once
 * per 128 nodes.
 */
size_t lm_head_q4_argmax_ws(int64_t n_rows, int64_t vocab, int64_t hidden_dim);
ttv_status lm_head_q4_argmax(const uint16_t* hidden, int64_t n_rows, int64_t hidden_stride, const uint32_t* wq,
                             const uint16_t* scale_bias, int64_t vocab, int64_t hidden_dim, int32_t* out_idx,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Step 4 -- accept walk [I1204] "What this needs" (2), "Increment 1"; [S728]
 * "What it does". Per tree: cur = 0, path = [0]; repeat: the child of cur
 * with the lowest label whose token equals target_argmax[cur] is appended and
 * becomes cur; stop when none matches. accepted = path_len - 1 and
 * emitted[k] = target_argmax[path[k]] (accepted + 1 tokens).
 *   parent, token, target_argmax (device) int32 [sum T_b] (tree-local labels)
 *   path     (device) int32 [B][64]  out (entries beyond path_len untouched)
 *   path_len (device) int32 [B]      out
 *   emitted  (device) int32 [B][64]  out
 *   sel      (device) int32 [B][sel_stride] out or NULL: the rollback
 *            selection [0, P_b) ++ (P_b + path[k]) ([PR1212] rollback-to-path
 *            commit), ready for kv_gather_positions with sel_len = path_len +
 *            P_b (written into sel_len_out when not NULL).
 *   sel_len_out (device) int32 [B] out or NULL
 * sel_stride must be >= max_b(P_b + T_b) when sel is given. An invalid
 * parent[] stores TTV_DEV_BAD_PARENT and writes nothing for that tree.
 */
ttv_status tree_accept_walk(const ttv_batch* batch, const int32_t* parent, const int32_t* token,
                            const int32_t* target_argmax, int32_t* path, int32_t* path_len,
                            int32_t* emitted, int32_t* sel, int32_t sel_stride, int32_t* sel_len_out,
                            int32_t* dev_status, void* stream);

/*
 * Step 5 -- rollback by gather along the sequence axis [I1204] "The rollback
 * constraint"; [PR1212] gather_positions commit, the commit widening it,
 * gather_within_tail commit. For every layer l, sequence b, head h and
 * j < sel_len[b]:
 *   dst.k[b][h][j] = src.k[b][h][sel[b][j]], likewise v and, for I8, the
 *   k_scale/v_scale sidecars (scales always move with their tokens).
 *   src, dst (host) arrays of n_layers descriptors. dst == NULL or every
 *            dst[l] describing the same buffers as src[l] means in place;
 *            otherwise dst must not overlap src. Shapes/dtypes must match.
 *   sel      (device) int32 [B][sel_stride], strictly increasing, each entry
 *            in [0, live_len_h[b]).
 *   sel_len  (device) int32 [B], 0 <= sel_len[b] <= live_len_h[b].
 *   live_len_h (host) int32 [B] current live rows per sequence.
 * All-or-nothing: a device-side check runs first; if any sequence's selection
 * is malformed, TTV_DEV_BAD_SELECTION is stored and no buffer is written.
 * In place, rows before the first j with sel[j] != j stay where they are, so an
 * identity or prefix selection (trim_to) moves 0 bytes and a tree rollback
 * moves only the accepted path's rows. Out of place, every survivor is written
 * (the pages' take). Rows at and beyond sel_len are not touched; the new live
 * length is sel_len[b].
 * ws: >= kv_gather_positions_ws(B) bytes.
 */
size_t kv_gather_positions_ws(int32_t B);
ttv_status kv_gather_positions(const ttv_kv_layer* src, const ttv_kv_layer* dst, int32_t n_layers,
                               int32_t B, const int32_t* sel, int32_t sel_stride,
                               const int32_t* sel_len, const int32_t* live_len_h,
                               int32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/*
 * Capability question asked before a tree is drafted [PR1212] the
 * tree_round_is_available and verify_finalize_tree commits: once the block is
 * on the cache a refusal has no recovery. Returns TTV_OK when every layer can
 * be verified as a tree and rolled back by kv_gather_positions, else
 * TTV_ERR_UNSUPPORTED (or TTV_ERR_INVALID) with the reason in ttv_last_error().
 * The gather moves rows of whole 16-byte pieces up to 4096 bytes (D * element
 * size; e.g. f32 up to D = 1024): wider rows, or an int8 cache without its
 * scale sidecars, are refused here and by every gather entry point.
 */
ttv_status kv_can_gather(const ttv_kv_layer* layers, int32_t n_layers);

/*
 * Tail form of step 5 for one verify block per sequence [PR1212] the
 * gather_within_tail commit (rewrite only the block's part of the window, so
 * the cost follows the block, not the context; the rotating form needs an
 * unwrapped ring and refuses by name once it has wrapped) and the commit
 * making the tail question "is it still in logical order". In place, for every
 * layer l, sequence b, head h and j < kept_len[b], with s = live_len_h[b] -
 * tail_len_h[b]:
 *   k[b][h][s + j] = k[b][h][s + kept[b][j]], likewise v and, for I8, the
 *   k_scale/v_scale sidecars.
 * The result equals kv_gather_positions in place with the absolute selection
 * [0, s) ++ (s + kept[b]); rows before the first j with kept[j] != j and rows
 * at and beyond s + kept_len[b] are not written; the new live length is
 * s + kept_len[b].
 *   layers      (host) n_layers descriptors (same shape and dtype).
 *   kept        (device) int32 [B][kept_stride], offsets inside the tail,
 *               strictly increasing, each in [0, tail_len_h[b]).
 *   kept_len    (device) int32 [B], 0 <= kept_len[b] <= tail_len_h[b].
 *   live_len_h  (host) int32 [B], current live rows (<= cap).
 *   tail_len_h  (host) int32 [B], the verify block's rows at the end of the
 *               live window, 0 <= tail_len <= min(live_len, 64).
 *   ring_wrapped_h (host) int32 [B] or NULL: nonzero when sequence b's cache
 *               is a rotating (sliding-window) ring that has wrapped, whose
 *               rows are then no longer in logical order; the call returns
 *               TTV_ERR_UNSUPPORTED naming the sequence and writes nothing.
 *               NULL: every cache keeps its rows in logical order (a linear
 *               cache, or a ring in the buffered regime that compacts from the
 *               front instead of wrapping).
 * All-or-nothing: a malformed kept/kept_len in any sequence stores
 * TTV_DEV_BAD_SELECTION and no buffer is written.
 * ws: >= kv_gather_within_tail_ws(B) bytes.
 */
size_t kv_gather_within_tail_ws(int32_t B);
ttv_status kv_gather_within_tail(const ttv_kv_layer* layers, int32_t n_layers, int32_t B, const int32_t* kept,
                                 int32_t kept_stride, const int32_t* kept_len, const int32_t* live_len_h,
                                 const int32_t* tail_len_h, const int32_t* ring_wrapped_h, int32_t* dev_status,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * Capability question for the tail form, answered from cache state (the
 * answer can change between rounds: a ring that wraps stops being gatherable)
 * [PR1212] the verify_finalize_tree and tree_round_is_available commits:
 * kv_can_gather(layers) and no sequence's ring wrapped. ring_wrapped_h as in
 * kv_gather_within_tail.
 */
ttv_status kv_can_gather_within_tail(const ttv_kv_layer* layers, int32_t n_layers, int32_t B,
                                     const int32_t* ring_wrapped_h);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* ttv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TTV_H */
