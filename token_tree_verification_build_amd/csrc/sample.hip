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
// Pass 1 streams the logits (HBM-bound): one wave per 4096-element chunk of a
// row, 64 ordered values per lane in registers. The chunk's top-k is found without a
// k-round scan over all of it: the k-th largest of the 64 lane maxima bounds
// the chunk's k-th largest value from below (k lanes hold a value at least
// that large), so only values at or above it are candidates; they are
// compacted into LDS (rarely more than a few dozen) and the top k taken there.
// Keys are 64-bit (ordered value << 32 | ~index), unique per element;
// selections run bit by bit on ballots and popcounts, with no lane shuffles.
// Pass 2 takes each row's top k from the chunks' candidates with one wave and
// makes the draw in float64: the exponentials one per lane, the running sums
// in descending order in one lane, the prefix and draw tests by ballot.
#include "common.hpp"

namespace ttv {

constexpr int kSampleMaxK = 64;
constexpr int kSampleLanes = 64;           // lanes per wave
constexpr int kSamplePerLane = 64;         // values per lane
constexpr int kSampleChunk = kSampleLanes * kSamplePerLane;  // 4096 values per wave
constexpr int kSampleWaves = 4;            // waves (chunks) per pass-1 workgroup
constexpr int kSampleCap = 256;            // candidate slots per wave in LDS
constexpr int kSampleMaxCand = 1 << 16;    // chunk candidates per row (pass 2 streams them)
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ordered key: larger value first, equal values by lower index; -0.0 folded
// onto +0.0, every NaN above every number
__device__ __forceinline__ uint64_t sample_key(float x, uint32_t idx) {
  uint32_t o;
  if (x != x) {
    o = 0xFFFFFFFFu;
  } else {
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0u) u = 0u;
    o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return 0xFFFFFFFFu - static_cast<uint32_t>(k); }
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = static_cast<uint32_t>(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Wave-wide selection without lane shuffles: the largest t such that at
// least `need` of the wave's keys (n per lane) are >= t, built bit by bit from
// the top (the count is non-increasing in t) with ballots and popcounts. For
// unique keys that is the need-th largest key; 0 when fewer than `need` are
// nonzero.
template <int N>
__device__ __forceinline__ uint64_t wave_kth_largest(const uint64_t (&key)[N], int need) {
  uint64_t t = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = t | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < N; ++s) cnt += __popcll(__ballot(key[s] >= cand));
    if (cnt >= need) t = cand;
  }
  return t;
}

// the lane's position among the set lanes of a wave-wide mask
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

// ordered 32-bit value (the key's high half): 0 only for "no value"
__device__ __forceinline__ uint32_t sample_ord(float x) { return static_cast<uint32_t>(sample_key(x, 0u) >> 32); }

// 32-bit form of wave_kth_largest (one value per lane)
__device__ __forceinline__ uint32_t wave_kth_largest32(uint32_t v, int need) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (__popcll(__ballot(v >= cand)) >= need) t = cand;
  }
  return t;
}

// Pass 1: wave w of workgroup (g, row) takes chunk c = 4g + w of the row and
// writes its top k keys (in no particular order; key 0, below every value,
// fills slots a short chunk cannot) to cand[(row * n_chunks + c) * k ...].
__global__ void __launch_bounds__(kSampleLanes * kSampleWaves)
    sample_pass1(const float* __restrict__ logits, int64_t vocab, int64_t row_stride, int n_chunks, int k, int vec,
                 uint64_t* __restrict__ cand) {
  __shared__ uint64_t s_cand[kSampleWaves][kSampleCap];
  const int wave = threadIdx.x / kSampleLanes;
  const int lane = threadIdx.x % kSampleLanes;
  const int row = blockIdx.y;
  const int c = blockIdx.x * kSampleWaves + wave;
  if (c >= n_chunks) return;  // whole wave; pass 1 has no workgroup barrier
  const float* __restrict__ x = logits + static_cast<int64_t>(row) * row_stride;
  const int64_t c0 = static_cast<int64_t>(c) * kSampleChunk;
  // the lane's ordered values: element c0 + 4 (64 j + lane) + q; past vocab 0
  uint32_t ov[kSamplePerLane];
  auto idx_of = [&](int j) -> uint32_t { return static_cast<uint32_t>(c0 + 4 * (64 * (j >> 2) + lane) + (j & 3)); };
  if (vec && c0 + kSampleChunk <= vocab) {
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x + c0);
#pragma unroll
    for (int j = 0; j < kSamplePerLane / 4; ++j) {
      const f32x4 a = __builtin_nontemporal_load(xv + 64 * j + lane);
      ov[4 * j] = sample_ord(a.x);
      ov[4 * j + 1] = sample_ord(a.y);
      ov[4 * j + 2] = sample_ord(a.z);
      ov[4 * j + 3] = sample_ord(a.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSamplePerLane; ++j) {
      const int64_t i = c0 + 4 * (64 * (j >> 2) + lane) + (j & 3);
      ov[j] = i < vocab ? sample_ord(x[i]) : 0u;
    }
  }
  // tau = the k-th largest lane maximum value, a lower bound on the chunk's
  // k-th largest value (k lanes hold a value at least that large); 0 when the
  // chunk holds fewer than k values
  uint32_t lmax = 0;
#pragma unroll
  for (int j = 0; j < kSamplePerLane; ++j) lmax = ov[j] > lmax ? ov[j] : lmax;
  const uint32_t tau = max(wave_kth_largest32(lmax, k), 1u);
  // compact the candidates' full keys (values >= tau) into LDS
  uint64_t* sc = s_cand[wave];
  int total = 0;
#pragma unroll
  for (int j = 0; j < kSamplePerLane; ++j) {
    const bool is = ov[j] >= tau;
    const uint64_t m = __ballot(is);
    if (m == 0) continue;  // (most steps: candidates are few)
    const int at = total + lanes_below(m);
    if (is && at < kSampleCap) sc[at] = (static_cast<uint64_t>(ov[j]) << 32) | (0xFFFFFFFFu - idx_of(j));
    total += __popcll(m);
  }
  uint64_t* out = cand + (static_cast<int64_t>(row) * n_chunks + c) * k;
  int n_out = 0;
  if (total <= kSampleCap) {
    __builtin_amdgcn_wave_barrier();
    // the k largest candidates: slots lane, lane + 64, ...
    uint64_t h[kSampleCap / kSampleLanes];
#pragma unroll
    for (int s = 0; s < kSampleCap / kSampleLanes; ++s) {
      const int at = lane + kSampleLanes * s;
      h[s] = at < total ? sc[at] : 0ull;
    }
    const uint64_t kth = wave_kth_largest(h, k);
#pragma unroll
    for (int s = 0; s < kSampleCap / kSampleLanes; ++s) {
      const bool is = h[s] != 0 && h[s] >= kth;
      const uint64_t m = __ballot(is);
      if (is) out[n_out + lanes_below(m)] = h[s];
      n_out += __popcll(m);
    }
  } else {
    // more candidates than slots (values tied near the bound): the same
    // selection over every value's full key, computed again
    uint64_t t = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cb = t | (1ull << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kSamplePerLane; ++j) {
        const uint64_t kj = ov[j] ? (static_cast<uint64_t>(ov[j]) << 32) | (0xFFFFFFFFu - idx_of(j)) : 0ull;
        cnt += __popcll(__ballot(kj >= cb));
      }
      if (cnt >= k) t = cb;
    }
#pragma unroll
    for (int j = 0; j < kSamplePerLane; ++j) {
      const uint64_t kj = ov[j] ? (static_cast<uint64_t>(ov[j]) << 32) | (0xFFFFFFFFu - idx_of(j)) : 0ull;
      const bool is = kj != 0 && kj >= t;
      const uint64_t m = __ballot(is);
      if (is) out[n_out + lanes_below(m)] = kj;
      n_out += __popcll(m);
    }
  }
  for (int i = n_out + lane; i < k; i += kSampleLanes) out[i] = 0;  // a chunk with fewer than k values
}

// Pass 2: one wave per row: the row's top k over its chunks' candidates (the
// same bound-and-compact scheme, streaming the candidates from the
// workspace), sorted descending by rank, then the draw (float64).
__global__ void __launch_bounds__(kSampleLanes) sample_pass2(const float* __restrict__ logits, int64_t row_stride,
                                                             const uint64_t* __restrict__ cand, int n_cand, int k,
                                                             const float* __restrict__ uniforms,
                                                             int64_t uniform_stride, float temperature, float top_p,
                                                             int32_t* __restrict__ out_idx) {
  __shared__ uint64_t s_c[kSampleCap];
  __shared__ uint64_t s_top[kSampleMaxK];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t* cr = cand + static_cast<int64_t>(row) * n_cand;
  auto cand_at = [&](int at) -> uint64_t { return at < n_cand ? cr[at] : 0ull; };
  // up to 64 * kRegCand candidates are held in registers (all loads in
  // flight at once); more are streamed, eight loads a step
  constexpr int kRegCand = 32;
  uint64_t lmax[1] = {0};
  int total = 0;
  uint64_t tau;
  if (n_cand <= kSampleLanes * kRegCand) {
    uint64_t v[kRegCand];
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) v[u] = cand_at(u * kSampleLanes + lane);
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) lmax[0] = v[u] > lmax[0] ? v[u] : lmax[0];
    tau = wave_kth_largest(lmax, k);
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) {
      const bool is = v[u] != 0 && v[u] >= tau;
      const uint64_t m = __ballot(is);
      const int at = total + lanes_below(m);
      if (is && at < kSampleCap) s_c[at] = v[u];
      total += __popcll(m);
    }
  } else {
    for (int base = 0; base < n_cand; base += 8 * kSampleLanes) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = cand_at(base + u * kSampleLanes + lane);
#pragma unroll
      for (int u = 0; u < 8; ++u) lmax[0] = v[u] > lmax[0] ? v[u] : lmax[0];
    }
    tau = wave_kth_largest(lmax, k);
    for (int base = 0; base < n_cand; base += 8 * kSampleLanes) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = cand_at(base + u * kSampleLanes + lane);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool is = v[u] != 0 && v[u] >= tau;
        const uint64_t m = __ballot(is);
        const int at = total + lanes_below(m);
        if (is && at < kSampleCap) s_c[at] = v[u];
        total += __popcll(m);
      }
    }
  }
  int n_w = 0;  // winners: the k largest keys (distinct, nonzero; the row has at least k values)
  if (total <= kSampleCap) {
    __builtin_amdgcn_wave_barrier();
    uint64_t g[kSampleCap / kSampleLanes];
#pragma unroll
    for (int s = 0; s < kSampleCap / kSampleLanes; ++s) {
      const int at = lane + kSampleLanes * s;
      g[s] = at < total ? s_c[at] : 0ull;
    }
    const uint64_t kth = wave_kth_largest(g, k);
#pragma unroll
    for (int s = 0; s < kSampleCap / kSampleLanes; ++s) {
      const bool is = g[s] != 0 && g[s] >= kth;
      const uint64_t m = __ballot(is);
      if (is) s_top[n_w + lanes_below(m)] = g[s];
      n_w += __popcll(m);
    }
  } else {
    // more candidates than slots (values tied near the bound): the same
    // bit-by-bit selection, counting over the streamed candidates
    uint64_t t = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cb = t | (1ull << bit);
      int cnt = 0;
      for (int base = 0; base < n_cand; base += kSampleLanes) cnt += __popcll(__ballot(cand_at(base + lane) >= cb));
      if (cnt >= k) t = cb;
    }
    for (int base = 0; base < n_cand; base += kSampleLanes) {
      const uint64_t v = cand_at(base + lane);
      const bool is = v != 0 && v >= t;
      const uint64_t m = __ballot(is);
      if (is) s_top[n_w + lanes_below(m)] = v;
      n_w += __popcll(m);
    }
  }
  __builtin_amdgcn_wave_barrier();
  // sort the k winners descending: each lane's rank is the count of larger keys
  const uint64_t mine = lane < k ? s_top[lane] : 0ull;
  int rank = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(mine)), j));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine >> 32), j));
    rank += ((static_cast<uint64_t>(hi) << 32) | lo) > mine ? 1 : 0;
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < k) s_top[rank] = mine;
  __builtin_amdgcn_wave_barrier();
  const uint64_t k0 = s_top[0];
  const float x0 = key_value(k0);
  if (x0 != x0 || x0 == INFINITY || x0 == -INFINITY) {  // a non-finite top logit is the selection
    if (lane == 0) out_idx[row] = static_cast<int32_t>(key_index(k0));
    return;
  }
  // exp(z_i - z_0) of the k winners, one per lane, then the running sums in
  // descending order by one lane
  __shared__ double s_e[kSampleMaxK];
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

static int sample_chunks(int64_t vocab) { return static_cast<int>((vocab + kSampleChunk - 1) / kSampleChunk); }

}  // namespace ttv

using namespace ttv;

extern "C" size_t vocab_sample_ws(int64_t n_rows, int64_t vocab, int32_t top_k) {
  if (n_rows <= 0 || vocab <= 0 || top_k <= 0) return 0;
  const int64_t k = top_k < vocab ? top_k : vocab;
  return static_cast<size_t>(n_rows) * sample_chunks(vocab) * k * sizeof(uint64_t);
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
  TTV_REQUIRE(top_k >= 1 && top_k <= kSampleMaxK, TTV_ERR_INVALID, "vocab_sample: top_k %d not in [1, %d]", top_k,
              kSampleMaxK);
  TTV_REQUIRE(temperature > 0.0f && temperature <= 3.0e38f, TTV_ERR_INVALID,
              "vocab_sample: temperature %g is not a positive finite number", (double)temperature);
  TTV_REQUIRE(top_p >= 0.0f && top_p <= 1.0f, TTV_ERR_INVALID, "vocab_sample: top_p %g not in [0, 1]",
              (double)top_p);
  TTV_REQUIRE(uniform_stride >= 0, TTV_ERR_INVALID, "vocab_sample: uniform_stride %lld < 0",
              (long long)uniform_stride);
  TTV_REQUIRE(logits && uniforms && out_idx, TTV_ERR_INVALID, "vocab_sample: NULL pointer");
  const int n_chunks = sample_chunks(vocab);
  const int k = static_cast<int>(top_k < vocab ? top_k : vocab);
  const int64_t n_cand = static_cast<int64_t>(n_chunks) * k;
  TTV_REQUIRE(n_cand <= kSampleMaxCand, TTV_ERR_INVALID,
              "vocab_sample: %d chunks x top_k %d candidates per row exceed %d (vocab too large for this top_k)",
              n_chunks, k, kSampleMaxCand);
  TTV_REQUIRE(n_rows <= 65535, TTV_ERR_INVALID, "vocab_sample: more than 65535 rows");
  const size_t need = vocab_sample_ws(n_rows, vocab, top_k);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "vocab_sample: workspace %zu bytes < %zu", ws_bytes, need);
  const int vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (row_stride % 4 == 0);
  hipStream_t s = (hipStream_t)stream;
  uint64_t* cand = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL(sample_pass1,
                     dim3(static_cast<unsigned>((n_chunks + kSampleWaves - 1) / kSampleWaves),
                          static_cast<unsigned>(n_rows)),
                     dim3(kSampleLanes * kSampleWaves), 0, s, logits, vocab, row_stride, n_chunks, k, vec, cand);
  ttv_status st = check_launch("vocab_sample pass 1");
  if (st != TTV_OK) return st;
  hipLaunchKernelGGL(sample_pass2, dim3(static_cast<unsigned>(n_rows)), dim3(kSampleLanes), 0, s, logits, row_stride,
                     static_cast<const uint64_t*>(cand), static_cast<int>(n_cand), k, uniforms, uniform_stride,
                     temperature, top_p, out_idx);
  return check_launch("vocab_sample pass 2");
}
