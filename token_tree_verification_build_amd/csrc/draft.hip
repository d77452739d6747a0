// Growing the draft tree from the drafter's confidence, the step before the
// mask: the branches go where the drafter is confident (EAGLE-2), using the
// drafter's per-step logits beyond their argmax ([I1204] "What this needs",
// the fourth decision; [PR1212] Drafter::draft_tree commit: the runner-up at
// an uncertain step is the alternative worth a verify position; [S728] "What
// it does": the chain plus alternatives from a top-k selector). Reading: the
// published EAGLE-2 expand-then-rerank procedure.
//
// A candidate's score is its float64 path log-probability (the sum of the
// drafter's log-softmax along the path). draft_tree_expand adds one depth:
// every frontier row's top_k tokens become children, and the next frontier
// is the top_k of those new candidates by score. draft_tree_select labels the
// root plus the n_nodes - 1 best candidates over all depths, best first.
//
// Expansion runs two launches. The first is the chunked top-k pass that also
// records each 4096-value chunk's maximum and float64 sum of exp(x - max) (so
// each logit is read from HBM once). The second uses one workgroup per
// sequence with one wave per frontier row: the row's top k from the chunk
// candidates, its log-normaliser from the chunk statistics (fixed reduction
// order, so identical rows give identical scores), the candidates' scores,
// and the next frontier by rank counting over the <= 256 new scores.
#include "topk.hpp"

namespace ttv {

constexpr int kDraftMaxK = 16;        // top_k limit: <= 16 frontier rows, <= 256 new candidates a depth
// chunks of 2,048 logits: twice the waves of 4,096-logit chunks, each half as
// long, which shortens the chunk pass more than the row pass's twice as many
// candidates lengthen it (1,024, 1,536, 3,072 and 4,096 were slower)
constexpr int kDraftPerLane = 32;
constexpr int kDraftChunk = kSelLanes * kDraftPerLane;
constexpr int kDraftMaxCand = 4096;   // candidate table limit per sequence

__device__ __forceinline__ bool draft_better(double su, int u, double st, int t) {
  return su > st || (su == st && u < t);
}

__global__ void __launch_bounds__(kSelLanes * kDraftMaxK)
    draft_expand_rows(const uint64_t* __restrict__ cand, int n_cand_row, const ChunkStats* __restrict__ stats,
                      int n_chunks, int k, int F, int depth, int32_t* __restrict__ cand_token,
                      int32_t* __restrict__ cand_parent, double* __restrict__ cand_score,
                      int32_t* __restrict__ cand_count, int cap, int32_t* __restrict__ frontier,
                      int32_t* __restrict__ dev_status) {
  __shared__ uint64_t s_c[kDraftMaxK][kSelCap];
  __shared__ uint64_t s_top[kDraftMaxK][kDraftMaxK];
  __shared__ double s_score[kDraftMaxK * kDraftMaxK];
  const int b = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kSelLanes));
  const int lane = threadIdx.x % kSelLanes;
  const int64_t base = static_cast<int64_t>(b) * cap;
  // The loads are ordered so that few of them wait on another: the table's
  // count, this wave's frontier slot and its parent's score are scalar
  // loads; the chunk statistics and candidates are vector loads issued
  // together. Nothing is written before every check has passed.
  const int n_old = depth == 1 ? 0 : cand_count[b];
  const int u = depth == 1 ? -1 : frontier[b * k + wave];
  // the table must hold a frontier to expand (slots in range) and room for F * k more
  const bool bad_state =
      (depth > 1 && (n_old < k || n_old > cap || u < 0 || u >= n_old)) || n_old + F * k > cap;
  const double pscore = (u >= 0 && !bad_state) ? cand_score[base + u] : 0.0;
  // the row's maximum and whether any value is not finite
  const int64_t row = static_cast<int64_t>(b) * F + wave;
  const ChunkStats* __restrict__ rs = stats + row * n_chunks;
  float m = -INFINITY;
  bool bad = false;
  for (int c = lane; c < n_chunks; c += kSelLanes) {
    const ChunkStats st = rs[c];
    bad |= st.bad != 0;
    m = st.max > m ? st.max : m;
  }
  // the row's top k, best first (into this wave's LDS only)
  row_topk_sorted(cand + row * n_cand_row, n_cand_row, k, lane, s_c[wave], s_top[wave]);
  const int any_state = __syncthreads_or(bad_state ? 1 : 0);
  const int any_logits = __syncthreads_or(bad ? 1 : 0);
  if (any_state || any_logits) {
    if (threadIdx.x == 0) *dev_status = any_state ? TTV_DEV_DRAFT_STATE : TTV_DEV_BAD_LOGITS;
    return;  // nothing written for this sequence
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  const double M = static_cast<double>(m);
  double S = 0.0;
  for (int c = lane; c < n_chunks; c += kSelLanes) {
    const ChunkStats st = rs[c];
    S += st.sum * exp_nonpos_f64(static_cast<double>(st.max) - M);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) S += __shfl_xor(S, off);
  const double lse = M + log(S);
  if (lane < k) {
    const uint64_t key = s_top[wave][lane];
    const double sc = pscore + (static_cast<double>(key_value(key)) - lse);
    const int at = n_old + wave * k + lane;
    cand_token[base + at] = static_cast<int32_t>(key_index(key));
    cand_parent[base + at] = u;
    cand_score[base + at] = sc;
    s_score[wave * k + lane] = sc;
  }
  __syncthreads();
  // next frontier: the k best of this depth's F * k candidates
  const int n_new = F * k;
  const int t = threadIdx.x;
  if (t < n_new) {
    const double st = s_score[t];
    int rank = 0;
    for (int v = 0; v < n_new; ++v) rank += draft_better(s_score[v], v, st, t) ? 1 : 0;
    if (rank < k) frontier[b * k + rank] = n_old + t;
  }
  if (t == 0) cand_count[b] = n_old + n_new;
}

__global__ void __launch_bounds__(1024)
    draft_select_nodes(int T, const int32_t* __restrict__ root_token, const int32_t* __restrict__ cand_token,
                       const int32_t* __restrict__ cand_parent, const double* __restrict__ cand_score,
                       const int32_t* __restrict__ cand_count, int cap, int32_t* __restrict__ parent,
                       int32_t* __restrict__ token, double* __restrict__ node_score, int32_t* __restrict__ dev_status) {
  __shared__ double s_sc[kDraftMaxCand];
  __shared__ int s_lab[kDraftMaxCand];
  __shared__ int s_err;
  const int b = blockIdx.x;
  const int64_t base = static_cast<int64_t>(b) * cap;
  const int n = cand_count[b];
  const int need = T - 1;
  if (n < need || n > cap) {
    if (threadIdx.x == 0) *dev_status = TTV_DEV_DRAFT_STATE;
    return;
  }
  if (threadIdx.x == 0) s_err = 0;
  for (int c = threadIdx.x; c < n; c += blockDim.x) s_sc[c] = cand_score[base + c];
  __syncthreads();
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const double sc = s_sc[c];
    int rank = 0;
    for (int v = 0; v < n; ++v) rank += draft_better(s_sc[v], v, sc, c) ? 1 : 0;
    s_lab[c] = rank < need ? rank + 1 : -1;
  }
  __syncthreads();
  // a chosen candidate's parent is chosen and labelled before it
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const int lab = s_lab[c];
    if (lab < 0) continue;
    const int u = cand_parent[base + c];
    if (u < -1 || u >= c || (u >= 0 && (s_lab[u] < 0 || s_lab[u] >= lab))) s_err = 1;
  }
  __syncthreads();
  if (s_err) {
    if (threadIdx.x == 0) *dev_status = TTV_DEV_DRAFT_STATE;
    return;
  }
  int32_t* __restrict__ po = parent + static_cast<int64_t>(b) * T;
  int32_t* __restrict__ to = token + static_cast<int64_t>(b) * T;
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const int lab = s_lab[c];
    if (lab < 0) continue;
    const int u = cand_parent[base + c];
    po[lab] = u < 0 ? 0 : s_lab[u];
    to[lab] = cand_token[base + c];
    if (node_score) node_score[static_cast<int64_t>(b) * T + lab] = s_sc[c];
  }
  if (threadIdx.x == 0) {
    po[0] = -1;
    to[0] = root_token[b];
    if (node_score) node_score[static_cast<int64_t>(b) * T] = 0.0;
  }
}

static size_t draft_ws_bytes(int64_t n_rows, int64_t vocab, int k) {
  const int64_t nc = sel_chunks(vocab, kDraftChunk);
  return static_cast<size_t>(n_rows * nc * k) * sizeof(uint64_t) + static_cast<size_t>(n_rows * nc) * sizeof(ChunkStats);
}

}  // namespace ttv

using namespace ttv;

extern "C" size_t draft_tree_expand_ws(int32_t n_rows, int64_t vocab, int32_t top_k) {
  if (n_rows <= 0 || vocab <= 0 || top_k <= 0) return 0;
  return draft_ws_bytes(n_rows, vocab, top_k);
}

extern "C" ttv_status draft_tree_expand(int32_t B, int32_t depth, int32_t top_k, const float* logits, int64_t vocab,
                                        int64_t row_stride, int32_t* cand_token, int32_t* cand_parent,
                                        double* cand_score, int32_t* cand_count, int32_t cand_cap, int32_t* frontier,
                                        int32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(B >= 1 && B <= TTV_MAX_BATCH, TTV_ERR_INVALID, "draft_tree_expand: B %d not in [1, %d]", B,
              TTV_MAX_BATCH);
  TTV_REQUIRE(depth >= 1, TTV_ERR_INVALID, "draft_tree_expand: depth %d < 1", depth);
  TTV_REQUIRE(top_k >= 1 && top_k <= kDraftMaxK, TTV_ERR_INVALID, "draft_tree_expand: top_k %d not in [1, %d]", top_k,
              kDraftMaxK);
  TTV_REQUIRE(vocab >= top_k && vocab <= 0x7FFFFFFF, TTV_ERR_INVALID,
              "draft_tree_expand: vocab %lld not in [top_k, 2^31 - 1]", (long long)vocab);
  TTV_REQUIRE(row_stride >= vocab, TTV_ERR_INVALID, "draft_tree_expand: row_stride %lld < vocab %lld",
              (long long)row_stride, (long long)vocab);
  TTV_REQUIRE(cand_cap >= top_k && cand_cap <= kDraftMaxCand, TTV_ERR_INVALID,
              "draft_tree_expand: cand_cap %d not in [top_k, %d]", cand_cap, kDraftMaxCand);
  TTV_REQUIRE(logits && cand_token && cand_parent && cand_score && cand_count && frontier && dev_status,
              TTV_ERR_INVALID, "draft_tree_expand: NULL pointer");
  const int F = depth == 1 ? 1 : top_k;
  const int64_t n_rows = static_cast<int64_t>(B) * F;
  const int n_chunks = sel_chunks(vocab, kDraftChunk);
  const int64_t n_cand_row = static_cast<int64_t>(n_chunks) * top_k;
  TTV_REQUIRE(n_cand_row <= kSelMaxCand, TTV_ERR_INVALID,
              "draft_tree_expand: %d chunks x top_k %d candidates per row exceed %d", n_chunks, top_k, kSelMaxCand);
  const size_t need = draft_ws_bytes(n_rows, vocab, top_k);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "draft_tree_expand: workspace %zu bytes < %zu", ws_bytes,
              need);
  const int vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (row_stride % 4 == 0);
  hipStream_t s = (hipStream_t)stream;
  uint64_t* cand = static_cast<uint64_t*>(ws);
  ChunkStats* stats = reinterpret_cast<ChunkStats*>(cand + n_rows * n_cand_row);
  hipLaunchKernelGGL((chunk_topk<true, kDraftPerLane>),
                     dim3(static_cast<unsigned>((n_chunks + kSelWaves - 1) / kSelWaves), static_cast<unsigned>(n_rows)),
                     dim3(kSelLanes * kSelWaves), 0, s, logits, vocab, row_stride, n_chunks, top_k, vec, cand, stats);
  ttv_status st = check_launch("draft_tree_expand chunk pass");
  if (st != TTV_OK) return st;
  hipLaunchKernelGGL(draft_expand_rows, dim3(static_cast<unsigned>(B)), dim3(kSelLanes * F), 0, s,
                     static_cast<const uint64_t*>(cand), static_cast<int>(n_cand_row),
                     static_cast<const ChunkStats*>(stats), n_chunks, top_k, F, depth, cand_token, cand_parent,
                     cand_score, cand_count, cand_cap, frontier, dev_status);
  return check_launch("draft_tree_expand rows");
}

extern "C" ttv_status draft_tree_select(int32_t B, int32_t n_nodes, const int32_t* root_token,
                                        const int32_t* cand_token, const int32_t* cand_parent,
                                        const double* cand_score, const int32_t* cand_count, int32_t cand_cap,
                                        int32_t* parent, int32_t* token, double* node_score, int32_t* dev_status,
                                        void* stream) {
  clear_error();
  TTV_REQUIRE(B >= 1 && B <= TTV_MAX_BATCH, TTV_ERR_INVALID, "draft_tree_select: B %d not in [1, %d]", B,
              TTV_MAX_BATCH);
  TTV_REQUIRE(n_nodes >= 1 && n_nodes <= TTV_MAX_NODES, TTV_ERR_INVALID, "draft_tree_select: n_nodes %d not in [1, %d]",
              n_nodes, TTV_MAX_NODES);
  TTV_REQUIRE(cand_cap >= 1 && cand_cap <= kDraftMaxCand, TTV_ERR_INVALID,
              "draft_tree_select: cand_cap %d not in [1, %d]", cand_cap, kDraftMaxCand);
  TTV_REQUIRE(root_token && cand_token && cand_parent && cand_score && cand_count && parent && token && dev_status,
              TTV_ERR_INVALID, "draft_tree_select: NULL pointer");
  hipLaunchKernelGGL(draft_select_nodes, dim3(static_cast<unsigned>(B)), dim3(1024), 0, (hipStream_t)stream, n_nodes,
                     root_token, cand_token, cand_parent, cand_score, cand_count, cand_cap, parent, token, node_score,
                     dev_status);
  return check_launch("draft_tree_select");
}
