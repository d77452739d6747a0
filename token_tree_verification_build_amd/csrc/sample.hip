// Sampled selection at every node, the temperature > 0 form of step 3: each
// node draws from the target's nucleus-filtered distribution with its own
// uniform ([S728] splash issue #728, "Historical issue and default question",
// "What it does": per-node uniforms at uniforms[n * uniform_stride], stride 0
// keeping one uniform for all; "Results": temperature 1, top-p 0.95, top-k 20).
// The filter chain: top-k by logit (ties to the lower index, the argmax
// order), float64 softmax of logit / temperature over those k summed in
// descending order, the shortest descending prefix whose cumulative mass
// reaches top-p, and the first kept token whose cumulative mass exceeds
// u times the prefix's mass.
//
// Pass 1 (chunk_topk, shared with the draft tree's expansion) streams the
// logits: one wave per 4096-element chunk of a row keeps the chunk's top k.
// Pass 2 takes each row's top k from the chunks' candidates with one wave and
// makes the draw in float64: the exponentials one per lane, the running sums
// in descending order in one lane, the prefix and draw tests by ballot.
#include "topk.hpp"

namespace ttv {

// Pass 2: one wave per row: the row's top k over its chunks' candidates (the
// same bound-and-compact scheme, streaming the candidates from the
// workspace), sorted descending by rank, then the draw (float64).
__global__ void __launch_bounds__(kSelLanes) sample_pass2(const float* __restrict__ logits, int64_t row_stride,
                                                         const uint64_t* __restrict__ cand, int n_cand, int k,
                                                         const float* __restrict__ uniforms, int64_t uniform_stride,
                                                         float temperature, float top_p,
                                                         int32_t* __restrict__ out_idx) {
  __shared__ uint64_t s_c[kSelCap];
  __shared__ uint64_t s_top[kSelMaxK];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  row_topk_sorted(cand + static_cast<int64_t>(row) * n_cand, n_cand, k, lane, s_c, s_top);
  const uint64_t k0 = s_top[0];
  const float x0 = key_value(k0);
  if (x0 != x0 || x0 == INFINITY || x0 == -INFINITY) {  // a non-finite top logit is the selection
    if (lane == 0) out_idx[row] = static_cast<int32_t>(key_index(k0));
    return;
  }
  // exp(z_i - z_0) of the k winners, one per lane, then the running sums in
  // descending order by one lane
  __shared__ double s_e[kSelMaxK];
  const float* __restrict__ xr = logits + static_cast<int64_t>(row) * row_stride;
  const double T = static_cast<double>(temperature);
  const double z0 = static_cast<double>(xr[key_index(k0)]) / T;
  if (lane < k) s_e[lane] = exp(static_cast<double>(xr[key_index(s_top[lane])]) / T - z0);
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {  // the running sums, in descending order
    double acc = 0.0;
    for (int i = 0; i < k; ++i) {
      acc += s_e[i];
      s_e[i] = acc;
    }
  }
  __builtin_amdgcn_wave_barrier();
  // C_i = c_i / c_{k-1} on lane i; the prefix end i* and the draw by ballots
  const double acc = s_e[k - 1];
  const double C = lane < k ? s_e[lane] / acc : 2.0;
  const uint64_t reach = __ballot(lane < k && C >= static_cast<double>(top_p));
  const int i_star = reach ? __builtin_ctzll(reach) : k - 1;
  const double c_star = __shfl(C, i_star);
  const double target = static_cast<double>(uniforms[static_cast<int64_t>(row) * uniform_stride]) * c_star;
  const uint64_t past = __ballot(lane <= i_star && C > target);
  const int pick = past ? __builtin_ctzll(past) : i_star;
  if (lane == 0) out_idx[row] = static_cast<int32_t>(key_index(s_top[pick]));
}

}  // namespace ttv

using namespace ttv;

extern "C" size_t vocab_sample_ws(int64_t n_rows, int64_t vocab, int32_t top_k) {
  if (n_rows <= 0 || vocab <= 0 || top_k <= 0) return 0;
  const int64_t k = top_k < vocab ? top_k : vocab;
  return static_cast<size_t>(n_rows) * sel_chunks(vocab) * k * sizeof(uint64_t);
}

extern "C" ttv_status vocab_sample(const float* logits, int64_t n_rows, int64_t vocab, int64_t row_stride,
                                   const float* uniforms, int64_t uniform_stride, float temperature, int32_t top_k,
                                   float top_p, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(n_rows >= 0 && vocab >= 1, TTV_ERR_INVALID, "vocab_sample: n_rows %lld, vocab %lld",
              (long long)n_rows, (long long)vocab);
  if (n_rows == 0) return TTV_OK;
  TTV_REQUIRE(vocab <= 0x7FFFFFFF, TTV_ERR_INVALID, "vocab_sample: vocab exceeds int32 indices");
  TTV_REQUIRE(row_stride >= vocab, TTV_ERR_INVALID, "vocab_sample: row_stride %lld < vocab %lld",
              (long long)row_stride, (long long)vocab);
  TTV_REQUIRE(top_k >= 1 && top_k <= kSelMaxK, TTV_ERR_INVALID, "vocab_sample: top_k %d not in [1, %d]", top_k,
              kSelMaxK);
  TTV_REQUIRE(temperature > 0.0f && temperature <= 3.0e38f, TTV_ERR_INVALID,
              "vocab_sample: temperature %g is not a positive finite number", (double)temperature);
  TTV_REQUIRE(top_p >= 0.0f && top_p <= 1.0f, TTV_ERR_INVALID, "vocab_sample: top_p %g not in [0, 1]",
              (double)top_p);
  TTV_REQUIRE(uniform_stride >= 0, TTV_ERR_INVALID, "vocab_sample: uniform_stride %lld < 0",
              (long long)uniform_stride);
  TTV_REQUIRE(logits && uniforms && out_idx, TTV_ERR_INVALID, "vocab_sample: NULL pointer");
  const int n_chunks = sel_chunks(vocab);
  const int k = static_cast<int>(top_k < vocab ? top_k : vocab);
  const int64_t n_cand = static_cast<int64_t>(n_chunks) * k;
  TTV_REQUIRE(n_cand <= kSelMaxCand, TTV_ERR_INVALID,
              "vocab_sample: %d chunks x top_k %d candidates per row exceed %d (vocab too large for this top_k)",
              n_chunks, k, kSelMaxCand);
  TTV_REQUIRE(n_rows <= 65535, TTV_ERR_INVALID, "vocab_sample: more than 65535 rows");
  const size_t need = vocab_sample_ws(n_rows, vocab, top_k);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "vocab_sample: workspace %zu bytes < %zu", ws_bytes, need);
  const int vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (row_stride % 4 == 0);
  hipStream_t s = (hipStream_t)stream;
  uint64_t* cand = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(chunk_topk<false>,
                     dim3(static_cast<unsigned>((n_chunks + kSelWaves - 1) / kSelWaves),
                          static_cast<unsigned>(n_rows)),
                     dim3(kSelLanes * kSelWaves), 0, s, logits, vocab, row_stride, n_chunks, k, vec, cand, nullptr);
  ttv_status st = check_launch("vocab_sample pass 1");
  if (st != TTV_OK) return st;
  hipLaunchKernelGGL(sample_pass2, dim3(static_cast<unsigned>(n_rows)), dim3(kSelLanes), 0, s, logits, row_stride,
                     static_cast<const uint64_t*>(cand), static_cast<int>(n_cand), k, uniforms, uniform_stride,
                     temperature, top_p, out_idx);
  return check_launch("vocab_sample pass 2");
}
