// Step 3 of a verify round: the target's greedy selection at every node, i.e.
// the lowest index of each logits row's maximum ([I1204] mlxcel issue #1204,
// "Increment 1": the target emits one argmax per position; [S728] splash issue
// #728, "Results": raw F32 argmax).
//
// HBM-bound streaming reduction. Each row is cut into chunks so that even a
// 3-node chain fills the GPU; a 256-thread workgroup scans one chunk with
// 16-byte loads, every thread keeping its own running (value, index) in index
// order, then reduces through wave shuffles and LDS with 64-bit keys
// (ordered value << 32 | ~index): the larger key is the larger value, and on
// equal values the lower index. Ordering: -0.0 is folded onto +0.0, every NaN
// maps to the largest key (so the first NaN wins). A second pass reduces the
// per-chunk keys of a row deterministically (no atomics).
#include "common.hpp"

namespace ttv {

constexpr int kArgThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t argmax_key(float x, int idx) {
  uint32_t o;
  if (x != x) {
    o = 0xFFFFFFFFu;
  } else {
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0u) u = 0u;  // -0.0 == +0.0
    o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

// Running best over elements seen in increasing index order: strictly greater
// wins (first occurrence kept), the first NaN wins and then sticks.
__device__ __forceinline__ void take(float x, int i, float& bv, int& bi) {
  if (bi < 0 || x > bv || (x != x && bv == bv)) {
    bv = x;
    bi = i;
  }
}

__device__ __forceinline__ uint64_t block_max_key(uint64_t key) {
  __shared__ uint64_t s_key[kArgThreads / kWave];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) s_key[w] = key;
  __syncthreads();
  uint64_t k = s_key[0];
#pragma unroll
  for (int i = 1; i < kArgThreads / kWave; ++i) k = s_key[i] > k ? s_key[i] : k;
  return k;
}

template <bool VEC>
__global__ void __launch_bounds__(kArgThreads) argmax_pass1(const float* __restrict__ logits, int64_t vocab,
                                                            int64_t row_stride, int64_t chunk, int n_chunks,
                                                            int32_t* __restrict__ out_idx,
                                                            uint64_t* __restrict__ keys) {
  const int row = blockIdx.x / n_chunks;
  const int c = blockIdx.x - row * n_chunks;
  const float* __restrict__ x = logits + static_cast<int64_t>(row) * row_stride;
  const int64_t lo = static_cast<int64_t>(c) * chunk;
  const int64_t hi = lo + chunk < vocab ? lo + chunk : vocab;
  float bv = 0.0f;
  int bi = -1;
  int64_t tail = lo;
  if constexpr (VEC) {
    const int64_t nvec = (hi - lo) >> 2;  // whole float4 groups in [lo, hi)
    const f32x4* __restrict__ xv = reinterpret_cast<const f32x4*>(x + lo);
    int64_t g = threadIdx.x;
    for (; g + 3 * kArgThreads < nvec; g += 4 * kArgThreads) {
      f32x4 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = __builtin_nontemporal_load(xv + g + u * kArgThreads);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int base = static_cast<int>(lo + 4 * (g + u * kArgThreads));
        take(a[u].x, base, bv, bi);
        take(a[u].y, base + 1, bv, bi);
        take(a[u].z, base + 2, bv, bi);
        take(a[u].w, base + 3, bv, bi);
      }
    }
    for (; g < nvec; g += kArgThreads) {
      const f32x4 a = __builtin_nontemporal_load(xv + g);
      const int base = static_cast<int>(lo + 4 * g);
      take(a.x, base, bv, bi);
      take(a.y, base + 1, bv, bi);
      take(a.z, base + 2, bv, bi);
      take(a.w, base + 3, bv, bi);
    }
    tail = lo + 4 * nvec;
  }
  for (int64_t i = tail + threadIdx.x; i < hi; i += kArgThreads) take(x[i], static_cast<int>(i), bv, bi);
  const uint64_t key = block_max_key(bi < 0 ? 0ull : argmax_key(bv, bi));
  if (threadIdx.x == 0) {
    if (n_chunks == 1)
      out_idx[row] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
    else
      keys[blockIdx.x] = key;
  }
}

__global__ void __launch_bounds__(kWave) argmax_pass2(const uint64_t* __restrict__ keys, int n_chunks,
                                                      int32_t* __restrict__ out_idx) {
  const int row = blockIdx.x;
  uint64_t k = 0;
  for (int i = threadIdx.x; i < n_chunks; i += kWave) {
    const uint64_t o = keys[static_cast<int64_t>(row) * n_chunks + i];
    k = o > k ? o : k;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  if (threadIdx.x == 0) out_idx[row] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k));
}

struct ArgmaxPlan {
  int n_chunks;
  int64_t chunk;
};

static ArgmaxPlan plan_argmax(int64_t n_rows, int64_t vocab) {
  // aim for >= 2048 workgroups, chunks of >= 2048 elements, 4-element aligned
  int64_t want = n_rows > 0 ? (2048 + n_rows - 1) / n_rows : 1;
  const int64_t max_chunks = (vocab + 2047) / 2048;
  if (want > max_chunks) want = max_chunks;
  if (want < 1) want = 1;
  int64_t chunk = (vocab + want - 1) / want;
  chunk = (chunk + 3) & ~int64_t(3);
  if (chunk < 4) chunk = 4;
  ArgmaxPlan p;
  p.chunk = chunk;
  p.n_chunks = static_cast<int>((vocab + chunk - 1) / chunk);
  return p;
}

}  // namespace ttv

using namespace ttv;

extern "C" size_t vocab_argmax_ws(int64_t n_rows, int64_t vocab) {
  if (n_rows <= 0 || vocab <= 0) return 0;
  const ArgmaxPlan p = plan_argmax(n_rows, vocab);
  return p.n_chunks > 1 ? static_cast<size_t>(n_rows) * p.n_chunks * sizeof(uint64_t) : 0;
}

extern "C" ttv_status vocab_argmax(const float* logits, int64_t n_rows, int64_t vocab, int64_t row_stride,
                                   int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(n_rows >= 0 && vocab >= 1, TTV_ERR_INVALID, "vocab_argmax: n_rows %lld, vocab %lld",
              (long long)n_rows, (long long)vocab);
  if (n_rows == 0) return TTV_OK;
  TTV_REQUIRE(vocab <= 0x7FFFFFFF, TTV_ERR_INVALID, "vocab_argmax: vocab exceeds int32 indices");
  TTV_REQUIRE(row_stride >= vocab, TTV_ERR_INVALID, "vocab_argmax: row_stride %lld < vocab %lld",
              (long long)row_stride, (long long)vocab);
  TTV_REQUIRE(logits && out_idx, TTV_ERR_INVALID, "vocab_argmax: NULL pointer");
  const ArgmaxPlan p = plan_argmax(n_rows, vocab);
  const size_t need = vocab_argmax_ws(n_rows, vocab);
  TTV_REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), TTV_ERR_WORKSPACE,
              "vocab_argmax: workspace %zu bytes < %zu", ws_bytes, need);
  const int64_t nblk = n_rows * p.n_chunks;
  TTV_REQUIRE(nblk <= 0x7FFFFFFF, TTV_ERR_INVALID, "vocab_argmax: too many rows");
  const bool vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (row_stride % 4 == 0);
  hipStream_t s = (hipStream_t)stream;
  if (vec)
    hipLaunchKernelGGL(argmax_pass1<true>, dim3(static_cast<unsigned>(nblk)), dim3(kArgThreads), 0, s, logits,
                       vocab, row_stride, p.chunk, p.n_chunks, out_idx, static_cast<uint64_t*>(ws));
  else
    hipLaunchKernelGGL(argmax_pass1<false>, dim3(static_cast<unsigned>(nblk)), dim3(kArgThreads), 0, s, logits,
                       vocab, row_stride, p.chunk, p.n_chunks, out_idx, static_cast<uint64_t*>(ws));
  ttv_status st = check_launch("vocab_argmax pass 1");
  if (st != TTV_OK || p.n_chunks == 1) return st;
  hipLaunchKernelGGL(argmax_pass2, dim3(static_cast<unsigned>(n_rows)), dim3(kWave), 0, s,
                     static_cast<const uint64_t*>(ws), p.n_chunks, out_idx);
  return check_launch("vocab_argmax pass 2");
}
