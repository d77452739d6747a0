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
// Pass 1 streams the logits (HBM-bound): one wave per 2048-element chunk of a
// row, 32 values per lane in registers. The chunk's top-k is found without a
// k-round scan over all of it: the k-th largest of the 64 lane maxima bounds
// the chunk's k-th largest value from below (k lanes hold a value at least
// that large), so only values at or above it are candidates; they are
// compacted into LDS (rarely more than a few dozen) and the top k taken there.
// Keys are 64-bit (ordered value << 32 | ~index), unique per element. Pass 2
// takes each row's top k from the chunks' candidates and makes the draw in
// one lane, in float64.
#include "common.hpp"

namespace ttv {

constexpr int kSampleMaxK = 64;
constexpr int kSampleLanes = 64;           // lanes per wave
constexpr int kSamplePerLane = 32;         // values per lane
constexpr int kSampleChunk = kSampleLanes * kSamplePerLane;  // 2048 values per wave
constexpr int kSampleWaves = 4;            // waves (chunks) per pass-1 workgroup
constexpr int kSampleCap = 256;            // candidate slots per wave in LDS
constexpr int kSampleMaxCand = 256 * 32;   // chunk candidates per row (pass 2 holds 32 per thread)
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  return k;
}

// Pass 1: wave w of workgroup (g, row) takes chunk c = 4g + w of the row and
// writes its top k keys, descending (key 0, below every value, fills slots a
// short chunk cannot), to cand[(row * n_chunks + c) * k ...].
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
  // the lane's values: element c0 + 4 (64 j + lane) + q, j < 8, q < 4; past
  // vocab they do not exist
  uint64_t kk[kSamplePerLane];  // the values' keys (0 past vocab: below every value)
  if (vec && c0 + kSampleChunk <= vocab) {
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x + c0);
#pragma unroll
    for (int j = 0; j < kSamplePerLane / 4; ++j) {
      const f32x4 a = __builtin_nontemporal_load(xv + 64 * j + lane);
      const uint32_t i0 = static_cast<uint32_t>(c0 + 4 * (64 * j + lane));
      kk[4 * j] = sample_key(a.x, i0);
      kk[4 * j + 1] = sample_key(a.y, i0 + 1);
      kk[4 * j + 2] = sample_key(a.z, i0 + 2);
      kk[4 * j + 3] = sample_key(a.w, i0 + 3);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSamplePerLane; ++j) {
      const int64_t i = c0 + 4 * (64 * (j >> 2) + lane) + (j & 3);
      kk[j] = i < vocab ? sample_key(x[i], static_cast<uint32_t>(i)) : 0ull;
    }
  }
  auto key_of = [&](int j) -> uint64_t { return kk[j]; };
  // the lane maximum and the k-th largest lane maximum: a lower bound tau on
  // the chunk's k-th largest key
  uint64_t lmax = 0;
#pragma unroll
  for (int j = 0; j < kSamplePerLane; ++j) {
    const uint64_t kj = key_of(j);
    lmax = kj > lmax ? kj : lmax;
  }
  uint64_t rest = lmax, tau = 0;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(rest);
    tau = m;
    if (rest == m) rest = 0;
  }
  // compact the candidates (keys >= tau; tau = 0 when the chunk holds fewer
  // than k values, then every value is one) into LDS
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kSamplePerLane; ++j) {
    const uint64_t kj = key_of(j);
    cnt += (kj != 0 && kj >= tau) ? 1 : 0;
  }
  int incl = cnt;  // inclusive prefix sum over the wave
#pragma unroll
  for (int off = 1; off < kSampleLanes; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int total = __shfl(incl, kSampleLanes - 1);
  uint64_t* out = cand + (static_cast<int64_t>(row) * n_chunks + c) * k;
  uint64_t* sc = s_cand[wave];
  if (total <= kSampleCap) {
    int at = incl - cnt;
#pragma unroll
    for (int j = 0; j < kSamplePerLane; ++j) {
      const uint64_t kj = key_of(j);
      if (kj != 0 && kj >= tau) sc[at++] = kj;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // top k of the candidates, largest first: each lane holds slots lane,
    // lane + 64, ... (up to 4)
    uint64_t h[kSampleCap / kSampleLanes];
#pragma unroll
    for (int s = 0; s < kSampleCap / kSampleLanes; ++s) {
      const int at2 = lane + kSampleLanes * s;
      h[s] = at2 < total ? sc[at2] : 0ull;
    }
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int s = 0; s < kSampleCap / kSampleLanes; ++s) best = h[s] > best ? h[s] : best;
      const uint64_t m = wave_max_u64(best);
      if (lane == 0) out[r] = m;
#pragma unroll
      for (int s = 0; s < kSampleCap / kSampleLanes; ++s)
        if (h[s] == m) h[s] = 0;  // keys are unique: one slot of one lane
    }
  } else {
    // more candidates than slots (many values tied near the bound): k rounds
    // over the lane's own values, exact and slower
    uint64_t lbest = lmax;
    for (int r = 0; r < k; ++r) {
      const uint64_t m = wave_max_u64(lbest);
      if (lane == 0) out[r] = m;
      if (lbest == m && m != 0) {  // this lane held it: drop it, rescan
        uint64_t nb = 0;
#pragma unroll
        for (int j = 0; j < kSamplePerLane; ++j) {
          const uint64_t kj = key_of(j);
          if (kj < m && kj > nb) nb = kj;
        }
        lbest = nb;
      }
    }
  }
}

// Pass 2: one workgroup per row: the row's top k over its chunks' candidates,
// then the draw in one lane (float64).
__global__ void __launch_bounds__(256) sample_pass2(const float* __restrict__ logits, int64_t row_stride,
                                                    const uint64_t* __restrict__ cand, int n_cand, int k,
                                                    const float* __restrict__ uniforms, int64_t uniform_stride,
                                                    float temperature, float top_p, int32_t* __restrict__ out_idx) {
  __shared__ uint64_t s_top[kSampleMaxK];
  __shared__ uint64_t s_wave[4];
  const int row = blockIdx.x;
  const int lane = threadIdx.x % kSampleLanes;
  const int wave = threadIdx.x / kSampleLanes;
  const uint64_t* cr = cand + static_cast<int64_t>(row) * n_cand;
  // candidates held per thread (n_cand <= 256 * H)
  constexpr int H = kSampleMaxCand / 256;
  uint64_t h[H];
#pragma unroll
  for (int s = 0; s < H; ++s) {
    const int at = static_cast<int>(threadIdx.x) + 256 * s;
    h[s] = at < n_cand ? cr[at] : 0ull;
  }
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int s = 0; s < H; ++s) best = h[s] > best ? h[s] : best;
    const uint64_t wm = wave_max_u64(best);
    if (lane == 0) s_wave[wave] = wm;
    __syncthreads();
    uint64_t m = s_wave[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) m = s_wave[q] > m ? s_wave[q] : m;
    if (threadIdx.x == 0) s_top[r] = m;
#pragma unroll
    for (int s = 0; s < H; ++s)
      if (h[s] == m) h[s] = 0;
    __syncthreads();  // s_wave is rewritten next round
  }
  if (threadIdx.x != 0) return;
  const uint64_t k0 = s_top[0];
  const float x0 = key_value(k0);
  if (x0 != x0 || x0 == INFINITY || x0 == -INFINITY) {  // a non-finite top logit is the selection
    out_idx[row] = static_cast<int32_t>(key_index(k0));
    return;
  }
  const float* __restrict__ xr = logits + static_cast<int64_t>(row) * row_stride;
  const double T = static_cast<double>(temperature);
  const double z0 = static_cast<double>(xr[key_index(k0)]) / T;
  auto e = [&](int i) { return exp(static_cast<double>(xr[key_index(s_top[i])]) / T - z0); };
  // running sums in descending order (recomputed per pass, identically)
  double acc = 0.0;
  for (int i = 0; i < k; ++i) acc += e(i);
  const double P = static_cast<double>(top_p);
  int i_star = k - 1;
  double c_star = acc;
  double c = 0.0;
  for (int i = 0; i < k; ++i) {
    c += e(i);
    if (c / acc >= P) {
      i_star = i;
      c_star = c;
      break;
    }
  }
  const double u = static_cast<double>(uniforms[static_cast<int64_t>(row) * uniform_stride]);
  const double target = u * (c_star / acc);
  int pick = i_star;
  c = 0.0;
  for (int i = 0; i <= i_star; ++i) {
    c += e(i);
    if (c / acc > target) {
      pick = i;
      break;
    }
  }
  out_idx[row] = static_cast<int32_t>(key_index(s_top[pick]));
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
  hipLaunchKernelGGL(sample_pass2, dim3(static_cast<unsigned>(n_rows)), dim3(256), 0, s, logits, row_stride,
                     static_cast<const uint64_t*>(cand), static_cast<int>(n_cand), k, uniforms, uniform_stride,
                     temperature, top_p, out_idx);
  return check_launch("vocab_sample pass 2");
}
