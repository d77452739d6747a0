// Chunked top-k selection over vocabulary rows, shared by the sampled target
// selection and the draft tree's expansion.
//
// Pass 1 streams the logits (HBM-bound): one wave per 4096-element chunk of a
// row, 64 ordered values per lane in registers. The chunk's top-k is found without a
// k-round scan over all of it: the k-th largest of the 64 lane maxima bounds
// the chunk's k-th largest value from below (k lanes hold a value at least
// that large), so only values at or above it are candidates; they are
// compacted into LDS (rarely more than a few dozen) and the top k taken there.
// Keys are 64-bit (ordered value << 32 | ~index), unique per element;
// selections run bit by bit on ballots and popcounts, with no lane shuffles.
// Optionally the same pass records each chunk's maximum and the float64 sum
// of exp(x - max), from which a row's log-normaliser follows.
// A row's top k over its chunks' candidates is then taken by one wave with
// the same bound-and-compact scheme (row_topk_sorted).
#pragma once

#include "common.hpp"

namespace ttv {

constexpr int kSelMaxK = 64;
constexpr int kSelLanes = 64;                         // lanes per wave
constexpr int kSelPerLane = 64;                       // values per lane (the default chunk)
constexpr int kSelChunk = kSelLanes * kSelPerLane;    // 4096 values per wave
constexpr int kSelWaves = 4;                          // waves (chunks) per pass-1 workgroup
constexpr int kSelCap = 256;                          // candidate slots per wave in LDS
constexpr int kSelMaxCand = 1 << 16;                  // chunk candidates per row (row_topk_sorted streams them)
typedef float f32x4 __attribute__((ext_vector_type(4)));

// per-chunk statistics of a row: max over the chunk, the float64 sum of
// exp(x - max), and whether any value is NaN or infinite
struct ChunkStats {
  double sum;
  float max;
  int bad;
};

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
// After the high 32 bits, if exactly `need` keys are >= t (no tie in the high
// halves at the boundary, the usual case), those are the `need` largest and
// the answer is their minimum, one wave reduction instead of 32 more steps.
template <int N>
__device__ __forceinline__ uint64_t wave_kth_largest(const uint64_t (&key)[N], int need) {
  uint64_t t = 0;
  for (int bit = 63; bit >= 32; --bit) {
    const uint64_t cand = t | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < N; ++s) cnt += __popcll(__ballot(key[s] >= cand));
    if (cnt >= need) t = cand;
  }
  int at_least = 0;
#pragma unroll
  for (int s = 0; s < N; ++s) at_least += __popcll(__ballot(key[s] >= t));
  if (at_least == need) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int s = 0; s < N; ++s) m = key[s] >= t && key[s] < m ? key[s] : m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = __shfl_xor(m, off);
      m = o < m ? o : m;
    }
    return m;
  }
  for (int bit = 31; bit >= 0; --bit) {
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

// e^t for t <= 0 in float64, a few ulp: Cody-Waite argument reduction
// t = n ln2 + r with |r| <= ln2 / 2 (ln2 split into a high part with
// trailing zero bits, so n * ln2_hi is exact, and a low part; the split of
// fdlibm), e^r by its Taylor series through r^13 (the next term is below
// 4e-18 relative) evaluated by Estrin's scheme (dependency depth 4 rather
// than 13, so the many exponentials of a wave overlap), scaled by 2^n with
// v_ldexp_f64 (subnormal results included); 0 below -745, under the
// smallest subnormal.
__device__ __forceinline__ double exp_nonpos_f64(double t) {
  if (t < -745.0) return 0.0;
  const double n = rint(t * 1.4426950408889634074);
  const double r = fma(-n, 1.90821492927058770002e-10, fma(-n, 6.93147180369123816490e-01, t));
  constexpr double f2 = 1.0 / 2, f3 = f2 / 3, f4 = f3 / 4, f5 = f4 / 5, f6 = f5 / 6, f7 = f6 / 7, f8 = f7 / 8,
                   f9 = f8 / 9, f10 = f9 / 10, f11 = f10 / 11, f12 = f11 / 12, f13 = f12 / 13;
  const double r2 = r * r;
  const double r4 = r2 * r2;
  const double r8 = r4 * r4;
  const double a0 = r + 1.0, a1 = fma(f3, r, f2), a2 = fma(f5, r, f4), a3 = fma(f7, r, f6);
  const double a4 = fma(f9, r, f8), a5 = fma(f11, r, f10), a6 = fma(f13, r, f12);
  const double b0 = fma(a1, r2, a0), b1 = fma(a3, r2, a2), b2 = fma(a5, r2, a4);
  const double d0 = fma(b1, r4, b0), d1 = fma(a6, r4, b2);
  return ldexp(fma(d1, r8, d0), static_cast<int>(n));
}

// The same exponential with a finer reduction, for the chunk statistics (one
// per logit): t = (64 q + j) ln2 / 64 + r with |r| <= ln2 / 128 (the same
// split of ln2, scaled by 1/64, so k * ln2_hi / 64 stays exact for |k| up to
// 2^21), e^t = 2^q * 2^(j/64) * e^r, e^r by its Taylor series through r^5 in
// Horner form (the next term is below 4e-17 relative), 2^(j/64) from a
// 64-entry table the caller fills with exp2_frac64 (a few ulp). About a third
// of the instructions of exp_nonpos_f64.
__device__ __forceinline__ double exp2_frac64(int j) {
  return 2.0 * exp_nonpos_f64(static_cast<double>(j - 64) * (6.93147180559945309417e-01 / 64.0));
}
__device__ __forceinline__ double exp_nonpos_tab(double t, const double* __restrict__ tab) {
  const double k = rint(t * (64.0 * 1.4426950408889634074));
  const double r = fma(-k, 1.90821492927058770002e-10 / 64.0, fma(-k, 6.93147180369123816490e-01 / 64.0, t));
  const int ki = static_cast<int>(k);
  constexpr double f3 = 1.0 / 6, f4 = f3 / 4, f5 = f4 / 5;
  const double e = fma(fma(fma(fma(fma(f5, r, f4), r, f3), r, 0.5), r, 1.0), r, 1.0);
  const double v = ldexp(tab[ki & 63] * e, ki >> 6);
  return t < -745.0 ? 0.0 : v;  // (k, and so ki, is not finite or out of range only here)
}

// Pass 1: wave w of workgroup (g, row) takes chunk c = 4g + w (of 64 *
// PER_LANE values) of the row and writes its top k keys (in no particular
// order; key 0, below every value, fills slots a short chunk cannot) to
// cand[(row * n_chunks + c) * k ...]. With kStats, lane 0 also writes the
// chunk's ChunkStats to stats[row * n_chunks + c].
template <bool kStats, int PER_LANE = kSelPerLane>
__global__ void __launch_bounds__(kSelLanes * kSelWaves)
    chunk_topk(const float* __restrict__ logits, int64_t vocab, int64_t row_stride, int n_chunks, int k, int vec,
               uint64_t* __restrict__ cand, ChunkStats* __restrict__ stats) {
  static_assert(PER_LANE % 4 == 0 && PER_LANE <= kSelPerLane, "chunk of 64 * PER_LANE values");
  constexpr int kChunk = kSelLanes * PER_LANE;
  __shared__ uint64_t s_cand[kSelWaves][kSelCap];
  __shared__ double s_exp_tab[kStats ? kSelWaves : 1][64];  // 2^(j/64), one copy per wave
  const int wave = threadIdx.x / kSelLanes;
  const int lane = threadIdx.x % kSelLanes;
  const int row = blockIdx.y;
  const int c = blockIdx.x * kSelWaves + wave;
  if (c >= n_chunks) return;  // whole wave; pass 1 has no workgroup barrier
  const double* tab = s_exp_tab[kStats ? wave : 0];
  if constexpr (kStats) {  // the wave's own table: its LDS writes precede its reads
    s_exp_tab[wave][lane] = exp2_frac64(lane);
    __builtin_amdgcn_wave_barrier();
  }
  const float* __restrict__ x = logits + static_cast<int64_t>(row) * row_stride;
  const int64_t c0 = static_cast<int64_t>(c) * kChunk;
  auto idx_of = [&](int j) -> uint32_t { return static_cast<uint32_t>(c0 + 4 * (64 * (j >> 2) + lane) + (j & 3)); };
  uint64_t* out = cand + (static_cast<int64_t>(row) * n_chunks + c) * k;
  if (vec && c0 + kChunk <= vocab) {
    // A full, aligned chunk: the values stay floats. The lane maxima, the
    // candidate test and the statistics run on them; only candidates become
    // ordered keys. x >= value(tau) is the same test as ord(x) >= tau for
    // every number (ord is monotone, -0.0 and +0.0 compare equal both ways),
    // and a NaN, which ranks above every number, is always a candidate.
    float xf[PER_LANE];
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x + c0);
#pragma unroll
    for (int j = 0; j < PER_LANE / 4; ++j) {
      const f32x4 a = __builtin_nontemporal_load(xv + 64 * j + lane);
      xf[4 * j] = a.x;
      xf[4 * j + 1] = a.y;
      xf[4 * j + 2] = a.z;
      xf[4 * j + 3] = a.w;
    }
    float lmf = -INFINITY, lmin = INFINITY;
    bool lnan = false;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      lmf = fmaxf(lmf, xf[j]);  // a NaN operand is skipped; NaNs are tracked apart
      lnan |= xf[j] != xf[j];
      if constexpr (kStats) lmin = fminf(lmin, xf[j]);
    }
    const uint32_t lmax = lnan ? 0xFFFFFFFFu : sample_ord(lmf);
    if constexpr (kStats) {
      uint32_t wm = lmax;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(wm), off));
        wm = o > wm ? o : wm;
      }
      const double m = static_cast<double>(key_value(static_cast<uint64_t>(wm) << 32));
      const bool bad = lnan || lmf == INFINITY || lmin == -INFINITY;
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < PER_LANE; ++j) sum += exp_nonpos_tab(static_cast<double>(xf[j]) - m, tab);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
      const bool any_bad = __ballot(bad) != 0;
      if (lane == 0) {
        ChunkStats st;
        st.sum = sum;
        st.max = static_cast<float>(m);
        st.bad = any_bad ? 1 : 0;
        stats[static_cast<int64_t>(row) * n_chunks + c] = st;
      }
    }
    const uint32_t tau = max(wave_kth_largest32(lmax, k), 1u);
    const float tau_f = key_value(static_cast<uint64_t>(tau) << 32);  // NaN when tau is the NaN rank
    auto fkey = [&](int j) -> uint64_t {
      return (static_cast<uint64_t>(sample_ord(xf[j])) << 32) | (0xFFFFFFFFu - idx_of(j));
    };
    uint64_t* sc = s_cand[wave];
    int total = 0;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      const bool is = xf[j] >= tau_f || xf[j] != xf[j];
      const uint64_t m = __ballot(is);
      if (m == 0) continue;
      const int at = total + lanes_below(m);
      if (is && at < kSelCap) sc[at] = fkey(j);
      total += __popcll(m);
    }
    int n_out = 0;
    if (total <= kSelLanes) {
      __builtin_amdgcn_wave_barrier();
      const uint64_t h1[1] = {lane < total ? sc[lane] : 0ull};
      const uint64_t kth = wave_kth_largest(h1, k);
      const bool is = h1[0] != 0 && h1[0] >= kth;
      const uint64_t m = __ballot(is);
      if (is) out[lanes_below(m)] = h1[0];
      n_out = __popcll(m);
    } else if (total <= kSelCap) {
      __builtin_amdgcn_wave_barrier();
      uint64_t h[kSelCap / kSelLanes];
#pragma unroll
      for (int q = 0; q < kSelCap / kSelLanes; ++q) {
        const int at = lane + kSelLanes * q;
        h[q] = at < total ? sc[at] : 0ull;
      }
      const uint64_t kth = wave_kth_largest(h, k);
#pragma unroll
      for (int q = 0; q < kSelCap / kSelLanes; ++q) {
        const bool is = h[q] != 0 && h[q] >= kth;
        const uint64_t m = __ballot(is);
        if (is) out[n_out + lanes_below(m)] = h[q];
        n_out += __popcll(m);
      }
    } else {
      // more candidates than slots (values tied near the bound): the
      // selection over every value's full key, computed again
      uint64_t t = 0;
      for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cb = t | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) cnt += __popcll(__ballot(fkey(j) >= cb));
        if (cnt >= k) t = cb;
      }
#pragma unroll
      for (int j = 0; j < PER_LANE; ++j) {
        const uint64_t kj = fkey(j);
        const bool is = kj >= t;
        const uint64_t m = __ballot(is);
        if (is) out[n_out + lanes_below(m)] = kj;
        n_out += __popcll(m);
      }
    }
    for (int i = n_out + lane; i < k; i += kSelLanes) out[i] = 0;  // (never: a full chunk holds k values)
    return;
  }
  // the lane's ordered values: element c0 + 4 (64 j + lane) + q; past vocab 0
  uint32_t ov[PER_LANE];
  {  // a ragged or unaligned chunk: ordered values, 0 past the vocabulary
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      const int64_t i = c0 + 4 * (64 * (j >> 2) + lane) + (j & 3);
      ov[j] = i < vocab ? sample_ord(x[i]) : 0u;
    }
  }
  // tau = the k-th largest lane maximum value, a lower bound on the chunk's
  // k-th largest value (k lanes hold a value at least that large); 0 when the
  // chunk holds fewer than k values
  uint32_t lmax = 0;
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) lmax = ov[j] > lmax ? ov[j] : lmax;
  if constexpr (kStats) {
    // chunk maximum; NaN orders as 0xFFFFFFFF, +inf as 0xFF800000 and -inf
    // as 0x007FFFFF, so those are the non-finite values
    uint32_t wm = lmax;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(wm), off));
      wm = o > wm ? o : wm;
    }
    const double m = static_cast<double>(key_value(static_cast<uint64_t>(wm) << 32));
    bool bad = false;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      bad |= ov[j] >= 0xFF800000u || ov[j] == 0x007FFFFFu;
      if (ov[j]) s += exp_nonpos_tab(static_cast<double>(key_value(static_cast<uint64_t>(ov[j]) << 32)) - m, tab);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const bool any_bad = __ballot(bad) != 0;
    if (lane == 0) {
      ChunkStats st;
      st.sum = s;
      st.max = static_cast<float>(m);
      st.bad = any_bad ? 1 : 0;
      stats[static_cast<int64_t>(row) * n_chunks + c] = st;
    }
  }
  const uint32_t tau = max(wave_kth_largest32(lmax, k), 1u);
  // compact the candidates' full keys (values >= tau) into LDS
  uint64_t* sc = s_cand[wave];
  int total = 0;
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) {
    const bool is = ov[j] >= tau;
    const uint64_t m = __ballot(is);
    if (m == 0) continue;  // (most steps: candidates are few)
    const int at = total + lanes_below(m);
    if (is && at < kSelCap) sc[at] = (static_cast<uint64_t>(ov[j]) << 32) | (0xFFFFFFFFu - idx_of(j));
    total += __popcll(m);
  }
  int n_out = 0;
  if (total <= kSelLanes) {
    // the usual case, a few dozen candidates: one slot per lane
    __builtin_amdgcn_wave_barrier();
    const uint64_t h1[1] = {lane < total ? sc[lane] : 0ull};
    const uint64_t kth = wave_kth_largest(h1, k);
    const bool is = h1[0] != 0 && h1[0] >= kth;
    const uint64_t m = __ballot(is);
    if (is) out[lanes_below(m)] = h1[0];
    n_out = __popcll(m);
  } else if (total <= kSelCap) {
    __builtin_amdgcn_wave_barrier();
    // the k largest candidates: slots lane, lane + 64, ...
    uint64_t h[kSelCap / kSelLanes];
#pragma unroll
    for (int s = 0; s < kSelCap / kSelLanes; ++s) {
      const int at = lane + kSelLanes * s;
      h[s] = at < total ? sc[at] : 0ull;
    }
    const uint64_t kth = wave_kth_largest(h, k);
#pragma unroll
    for (int s = 0; s < kSelCap / kSelLanes; ++s) {
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
      for (int j = 0; j < PER_LANE; ++j) {
        const uint64_t kj = ov[j] ? (static_cast<uint64_t>(ov[j]) << 32) | (0xFFFFFFFFu - idx_of(j)) : 0ull;
        cnt += __popcll(__ballot(kj >= cb));
      }
      if (cnt >= k) t = cb;
    }
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      const uint64_t kj = ov[j] ? (static_cast<uint64_t>(ov[j]) << 32) | (0xFFFFFFFFu - idx_of(j)) : 0ull;
      const bool is = kj != 0 && kj >= t;
      const uint64_t m = __ballot(is);
      if (is) out[n_out + lanes_below(m)] = kj;
      n_out += __popcll(m);
    }
  }
  for (int i = n_out + lane; i < k; i += kSelLanes) out[i] = 0;  // a chunk with fewer than k values
}

// One wave: the k largest of a row's n_cand chunk candidates cr[0..n_cand)
// (the same bound-and-compact scheme, streaming the candidates), sorted
// descending into s_top[0..k). s_c is kSelCap slots of LDS scratch. The row
// must hold at least k values.
__device__ __forceinline__ void row_topk_sorted(const uint64_t* __restrict__ cr, int n_cand, int k, int lane,
                                                uint64_t* s_c, uint64_t* s_top) {
  auto cand_at = [&](int at) -> uint64_t { return at < n_cand ? cr[at] : 0ull; };
  // up to 64 * kRegCand candidates are held in registers (all loads in
  // flight at once); more are streamed, eight loads a step
  constexpr int kRegCand = 32;
  uint64_t lmax[1] = {0};
  int total = 0;
  uint64_t tau;
  if (n_cand <= kSelLanes * kRegCand) {
    uint64_t v[kRegCand];
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) v[u] = cand_at(u * kSelLanes + lane);
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) lmax[0] = v[u] > lmax[0] ? v[u] : lmax[0];
    tau = wave_kth_largest(lmax, k);
#pragma unroll
    for (int u = 0; u < kRegCand; ++u) {
      const bool is = v[u] != 0 && v[u] >= tau;
      const uint64_t m = __ballot(is);
      const int at = total + lanes_below(m);
      if (is && at < kSelCap) s_c[at] = v[u];
      total += __popcll(m);
    }
  } else {
    for (int base = 0; base < n_cand; base += 8 * kSelLanes) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = cand_at(base + u * kSelLanes + lane);
#pragma unroll
      for (int u = 0; u < 8; ++u) lmax[0] = v[u] > lmax[0] ? v[u] : lmax[0];
    }
    tau = wave_kth_largest(lmax, k);
    for (int base = 0; base < n_cand; base += 8 * kSelLanes) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = cand_at(base + u * kSelLanes + lane);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool is = v[u] != 0 && v[u] >= tau;
        const uint64_t m = __ballot(is);
        const int at = total + lanes_below(m);
        if (is && at < kSelCap) s_c[at] = v[u];
        total += __popcll(m);
      }
    }
  }
  int n_w = 0;  // winners: the k largest keys (distinct, nonzero; the row has at least k values)
  if (total <= kSelLanes) {
    __builtin_amdgcn_wave_barrier();
    const uint64_t g1[1] = {lane < total ? s_c[lane] : 0ull};
    const uint64_t kth = wave_kth_largest(g1, k);
    const bool is = g1[0] != 0 && g1[0] >= kth;
    const uint64_t m = __ballot(is);
    if (is) s_top[lanes_below(m)] = g1[0];
    n_w = __popcll(m);
  } else if (total <= kSelCap) {
    __builtin_amdgcn_wave_barrier();
    uint64_t g[kSelCap / kSelLanes];
#pragma unroll
    for (int s = 0; s < kSelCap / kSelLanes; ++s) {
      const int at = lane + kSelLanes * s;
      g[s] = at < total ? s_c[at] : 0ull;
    }
    const uint64_t kth = wave_kth_largest(g, k);
#pragma unroll
    for (int s = 0; s < kSelCap / kSelLanes; ++s) {
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
      for (int base = 0; base < n_cand; base += kSelLanes) cnt += __popcll(__ballot(cand_at(base + lane) >= cb));
      if (cnt >= k) t = cb;
    }
    for (int base = 0; base < n_cand; base += kSelLanes) {
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
}

inline int sel_chunks(int64_t vocab, int chunk = kSelChunk) { return static_cast<int>((vocab + chunk - 1) / chunk); }

}  // namespace ttv
