// The LM-head projection fused with the greedy selection: the target's logit
// row of every node is the product of its final hidden state with the head
// weight, and at temperature 0 the row exists only for its argmax ([I1185]
// mlxcel issue #1185, "Proposed work", Phase 2a: a fused projection-plus-
// argmax kernel never writes the logits). Ties go to the lowest index, as in
// vocab_argmax (-0.0 equals +0.0, a NaN outranks every number).
//
// Operands: hidden states X [N][H] and the head weight W [V][H] (one
// vocabulary row per H-vector), both bf16; fp32 accumulation on the matrix
// cores (v_mfma_f32_16x16x32_bf16: bf16 x bf16 products are exact in fp32).
// The weight dominates the bytes (V * H * 2), each element is used by one
// wave only, so it goes straight from HBM to registers: a wave owns 64
// vocabulary rows (four 16-row blocks) and streams them along H, 128
// contiguous bytes per row per 64-element step, the next step's loads in
// flight while the current one multiplies. The hidden states are shared by
// the workgroup's 8 waves and staged through LDS in 64-element slices
// (double buffered, rows padded against bank conflicts). With lane = (i =
// lane % 16, g = lane / 16): A = W block (16 rows x 32 k, lane (i, g) holds
// row i, k = 8g .. 8g+7), B = X block transposed (lane (i, g) holds node i's
// k = 8g .. 8g+7), and the output lane (i, g) holds vocabulary rows 4g .. 4g+3
// of node i. A workgroup covers 512 rows x up to 128 nodes; more nodes take
// more node slices (each re-reads the weight; slices of one vocabulary slab
// are dealt to the same XCD back to back so the re-reads tend to hit L2).
// The epilogue reduces each node's 64-bit keys (ordered logit << 32 | ~index)
// over the wave's rows, the workgroup's waves, and finally, in a second
// launch, over the vocabulary slabs.
#include "common.hpp"

namespace ttv {

constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kLmMaxVB = 4;                              // blocks of 16 vocabulary rows per wave, at most
constexpr int kLmKc = 64;                                // k elements per LDS slice (two MFMA steps)
constexpr int kLmXPitch = kLmKc * 2 + 16;                // bytes per staged hidden row (padded)
constexpr int kLmMaxNB = 8;                              // 16-node blocks per slice (128 nodes)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t lm_key(float x, uint32_t idx) {
  uint32_t o;
  if (x != x) {
    o = 0xFFFFFFFFu;
  } else {
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0u) u = 0u;  // -0.0 == +0.0
    o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - idx);
}

struct LmParams {
  const uint16_t* x;    // [N][x_stride] bf16
  const uint16_t* w;    // [V][w_stride] bf16
  uint64_t* part;       // [N][n_slabs] best key per (node, slab)
  int64_t x_stride;
  int64_t w_stride;
  int N, V, H;
  int n_slabs, n_slices;
};

// A wave owns VB blocks of 16 vocabulary rows (VB = 4 up to 112 nodes; at
// 128 only 3 fit beside the accumulators, both weight slots and the hidden
// fragments in 256 registers, and 2 run ~1% faster than 3: 970 workgroups
// fill the last round better than 647), a workgroup kLmWaves * 16 * VB rows.
template <int NB, int VB>
__global__ void __launch_bounds__(kLmThreads) lm_head_main(const LmParams p) {
  constexpr int kRows = 16 * VB;
  __shared__ __attribute__((aligned(16))) unsigned char s_x[2][16 * NB * kLmXPitch];
  __shared__ uint64_t s_best[kLmWaves][16 * NB];
  const int slot = xcd_slot(blockIdx.x, p.n_slabs * p.n_slices);
  if (slot < 0) return;  // padding workgroup (whole block, before any barrier)
  const int slab = slot / p.n_slices;
  const int slice = slot % p.n_slices;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  const int lane = threadIdx.x % kWave;
  const int li = lane % 16, lg = lane / 16;
  const int n0 = slice * 16 * kLmMaxNB;
  const int v_wave = slab * kLmWaves * kRows + wave * kRows;

  // weight rows of this lane (clamped into range; rows past V are ignored)
  const unsigned char* wrow[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    const int v = min(v_wave + 16 * vb + li, p.V - 1);
    wrow[vb] = reinterpret_cast<const unsigned char*>(p.w + static_cast<int64_t>(v) * p.w_stride) + 16 * lg;
  }
  // hidden-state staging: piece t = threadIdx.x + 512 r covers row t / 8,
  // bytes 16 (t % 8) of the slice
  constexpr int kPieces = 16 * NB * 8;
  constexpr int kPiecesPerThread = (kPieces + kLmThreads - 1) / kLmThreads;
  auto x_piece = [&](int c, int r) -> u32x4 {
    const int t = threadIdx.x + kLmThreads * r;
    const int row = min(n0 + t / 8, p.N - 1);
    const unsigned char* src = reinterpret_cast<const unsigned char*>(p.x + static_cast<int64_t>(row) * p.x_stride) +
                               c * (kLmKc * 2) + 16 * (t % 8);
    return *reinterpret_cast<const u32x4*>(src);
  };
  auto x_store = [&](int buf, int r, u32x4 v) {
    const int t = threadIdx.x + kLmThreads * r;
    *reinterpret_cast<u32x4*>(&s_x[buf][(t / 8) * kLmXPitch + 16 * (t % 8)]) = v;
  };

  f32x4 acc[VB][NB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[vb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_chunks = p.H / kLmKc;
  const int last = n_chunks - 1;
  // Weight fragments in a two-slot register ring: slot c & 1 holds slice c's
  // and is refilled with slice c + 2's as soon as slice c's MFMAs have been
  // issued, so no loaded register is copied from one slice to the next (a
  // copy of a register still loading would wait for that load, exposing its
  // latency every slice). The slice loop is unrolled by two so that the slot
  // index is known at compile time; past the last slice the refill re-reads
  // it (in bounds, never used).
  u32x4 wr[2][2][VB];
  auto w_load = [&](int c, int h, int vb) {
    return *reinterpret_cast<const u32x4*>(wrow[vb] + c * (kLmKc * 2) + 64 * h);
  };
  // prologue: slice 0 of the hidden states into LDS, weight slices 0 and 1 in flight
  u32x4 xs[kPiecesPerThread];
#pragma unroll
  for (int r = 0; r < kPiecesPerThread; ++r)
    if (threadIdx.x + kLmThreads * r < kPieces) xs[r] = x_piece(0, r);
#pragma unroll
  for (int r = 0; r < kPiecesPerThread; ++r)
    if (threadIdx.x + kLmThreads * r < kPieces) x_store(0, r, xs[r]);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) wr[q][h][vb] = w_load(min(q, last), h, vb);
  __syncthreads();

  auto step = [&](int c, auto slot_tag) __attribute__((always_inline)) {
    constexpr int Q = decltype(slot_tag)::value;  // == c & 1
    const int buf = Q;
    const bool more = c + 1 < n_chunks;
    // next slice's hidden pieces in flight
    if (more) {
#pragma unroll
      for (int r = 0; r < kPiecesPerThread; ++r)
        if (threadIdx.x + kLmThreads * r < kPieces) xs[r] = x_piece(c + 1, r);
    }
    // two 32-k steps on the current slice, one hidden fragment at a time:
    // fragment f + 1 is read while fragment f multiplies, and a scheduling
    // barrier closes each fragment, so the compiler cannot hoist all the
    // reads (their registers would not fit beside the accumulators and both
    // weight slots)
    auto x_frag = [&](int f) {
      const int h = f / NB, nb = f % NB;
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(&s_x[buf][(16 * nb + li) * kLmXPitch + 64 * h + 16 * lg]));
    };
    bf16x8 xf = x_frag(0);
#pragma unroll
    for (int f = 0; f < 2 * NB; ++f) {
      const int h = f / NB, nb = f % NB;
      const bf16x8 xn = f + 1 < 2 * NB ? x_frag(f + 1) : xf;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
        acc[vb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wr[Q][h][vb]), xf,
                                                              acc[vb][nb], 0, 0, 0);
      xf = xn;
      __builtin_amdgcn_sched_barrier(0);
    }
    // the slot refilled with slice c + 2
    const int c2 = min(c + 2, last);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) wr[Q][h][vb] = w_load(c2, h, vb);
    if (more) {
#pragma unroll
      for (int r = 0; r < kPiecesPerThread; ++r)
        if (threadIdx.x + kLmThreads * r < kPieces) x_store(buf ^ 1, r, xs[r]);
    }
    __syncthreads();
  };
  int c = 0;
  for (; c + 1 < n_chunks; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    step(c + 1, std::integral_constant<int, 1>{});
  }
  if (c < n_chunks) step(c, std::integral_constant<int, 0>{});

  // epilogue: node 16 nb + li's best over the lane's rows 16 vb + 4 lg + j
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    uint64_t best = 0;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = v_wave + 16 * vb + 4 * lg + j;
        if (v < p.V) {
          const uint64_t k = lm_key(acc[vb][nb][j], static_cast<uint32_t>(v));
          best = k > best ? k : best;
        }
      }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const uint64_t o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
    if (lg == 0) s_best[wave][16 * nb + li] = best;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 16 * NB && n0 + t < p.N) {
    uint64_t best = s_best[0][t];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w) best = s_best[w][t] > best ? s_best[w][t] : best;
    p.part[static_cast<int64_t>(n0 + t) * p.n_slabs + slab] = best;
  }
}

// The 4-bit head ([I1185] "The cost model": the borrowed head is 248,320 x
// 5,120 codes + a scale and a bias per 64-element group; the "Phase 3 done"
// comment: affine group-64 4-bit). Value = scale * code + bias, code 0..15,
// 8 codes per 32-bit word (hidden element i in bits 4 (i mod 8) of word
// i / 8), (scale, bias) bf16 pairs stored group-major [H/64][V][2].
//
// logit(v, n) = sum_g scale[g][v] * (sum_{i in g} code[v][i] x[n][i])
//             + sum_g bias[g][v] * X[n][g],   X[n][g] = sum_{i in g} x[n][i].
//
// Same tiling as the bf16 kernel (a wave owns VB * 16 vocabulary rows, the
// hidden states are staged through LDS one 64-element group at a time), but
// each 32-k MFMA step stays inside one group: lane (i, g) takes hidden
// elements 64 gi + 8 (2g + h) .. +8 in step h, i.e. code words 8 gi + 2g and
// 8 gi + 2g + 1 (one 8-byte load). Codes become bf16 small integers exactly,
// each group's products accumulate from zero on the matrix cores and the
// group is folded in as acc += scale * partial. The bias term is a small
// product of its own (vocabulary x groups times groups x nodes) on the matrix
// cores, 32 groups at a time: a first launch forms X in fp32 and splits it
// exactly into three bf16 terms (hi + mid + lo), so its products are exact
// and accumulate in fp32 onto acc. The biases arrive with the scales; each
// wave keeps its rows' biases of the current and the next 32 groups in LDS,
// and the group sums of a chunk are staged in LDS with its last group.
// A wave holds VB * 16 = 32 vocabulary rows x NB * 16 nodes (NB <= 8), so up
// to 128 nodes share one slice: every code is converted once for all of them
// and the head is read once. The group's partial sums are formed one node
// block at a time, the fold of each block issued in the shadow of the next
// block's MFMAs, so only two blocks of partial sums are live. Workgroups are
// 8 waves (256 vocabulary rows).
constexpr int kLmQ4MaxNB = 8;
constexpr int kLmQ4Slab = 256;                             // vocabulary rows per workgroup, for the workspace
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// byte B of x as a float (v_cvt_f32_ubyte<B>: one instruction, where the
// compiler otherwise extracts the byte first)
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  float f;
  if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(x));
  else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
  else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(x));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(x));
  return f;
}

// 8 codes of one word as bf16x8: small integers are exact in bf16, so a
// float's top half is the bf16; one byte permute packs two of them
__device__ __forceinline__ u32x4 q4_to_bf16x8(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(__float_as_uint(ubyte_f32<0>(hi)), __float_as_uint(ubyte_f32<0>(lo)), 0x07060302u);
  r[1] = __builtin_amdgcn_perm(__float_as_uint(ubyte_f32<1>(hi)), __float_as_uint(ubyte_f32<1>(lo)), 0x07060302u);
  r[2] = __builtin_amdgcn_perm(__float_as_uint(ubyte_f32<2>(hi)), __float_as_uint(ubyte_f32<2>(lo)), 0x07060302u);
  r[3] = __builtin_amdgcn_perm(__float_as_uint(ubyte_f32<3>(hi)), __float_as_uint(ubyte_f32<3>(lo)), 0x07060302u);
  return r;
}

struct LmQ4Params {
  const uint16_t* x;    // [N][x_stride] bf16
  const uint32_t* wq;   // [V][H/8] packed codes
  const uint16_t* sb;   // [H/64][V][2] bf16 (scale, bias)
  uint64_t* part;       // [N][n_slabs]
  const uint16_t* xg;   // [3][N][Gp] bf16: the group sums' hi, mid and lo terms (zero for g >= G)
  int64_t x_stride;
  int N, V, H;
  int Gp;               // groups rounded up to a multiple of 32
  int n_slabs, n_slices;
};

// X[n][g] in fp32 (the group's 64 values in order), split exactly into
// hi + mid + lo with each term a bf16 (truncation leaves a remainder of at
// most 16, then 8 significant bits); padded groups g in [G, Gp) are zero.
__global__ void __launch_bounds__(256) lm_q4_group_sums(const uint16_t* __restrict__ x, int64_t x_stride, int N,
                                                       int G, int Gp, uint16_t* __restrict__ xg) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= static_cast<int64_t>(N) * Gp) return;
  const int n = static_cast<int>(t / Gp), g = static_cast<int>(t % Gp);
  float s = 0.f;
  if (g < G) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + n * x_stride + 64 * g);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 v = src[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += __uint_as_float(v[e] << 16);
        s += __uint_as_float(v[e] & 0xFFFF0000u);
      }
    }
  }
  const uint32_t hi = __float_as_uint(s) & 0xFFFF0000u;
  const float r1 = s - __uint_as_float(hi);
  const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mid);
  const size_t plane = static_cast<size_t>(N) * Gp;
  xg[t] = static_cast<uint16_t>(hi >> 16);
  xg[plane + t] = static_cast<uint16_t>(mid >> 16);
  xg[2 * plane + t] = static_cast<uint16_t>(__float_as_uint(r2) >> 16);
}

template <int NB, int NW, int VB>
__global__ void __launch_bounds__(NW * kWave) lm_head_q4_main(const LmQ4Params p) {
  static_assert(VB * NB <= 16 && NW * VB * 16 == kLmQ4Slab, "accumulators, slab");
  constexpr int kLmQ4Threads = NW * kWave;
  constexpr int kSlab = NW * VB * 16;
  constexpr int kRows = VB * 16;  // vocabulary rows per wave
  __shared__ __attribute__((aligned(16))) unsigned char s_x[2][16 * NB * kLmXPitch];
  // biases of the wave's rows for groups g (slot g % 64): two chunks of 32
  __shared__ __attribute__((aligned(16))) uint16_t s_bias[NW][64][kRows];
  // the group sums' three bf16 terms of the current chunk of 32 groups:
  // [term][node row] rows of 64 bytes, padded to kXgPitch (conflict-free
  // 16-byte reads by 16 consecutive node rows), filled by whole 1 KiB
  // direct-to-LDS loads
  constexpr int kXgPitch = 80;
  constexpr int kXgRows = 3 * 16 * NB;
  constexpr int kXgSlots = kXgRows * (kXgPitch / 16);  // 16-byte slots
  constexpr int kXgDma = (kXgSlots + 63) / 64;         // loads of 64 slots
  __shared__ __attribute__((aligned(16))) unsigned char s_xg[kXgDma * 1024];
  __shared__ uint64_t s_best[NW][16 * NB];
  const int slot = xcd_slot(blockIdx.x, p.n_slabs * p.n_slices);
  if (slot < 0) return;  // padding workgroup (whole block, before any barrier)
  const int slab = slot / p.n_slices;
  const int slice = slot % p.n_slices;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  const int lane = threadIdx.x % kWave;
  const int li = lane % 16, lg = lane / 16;
  const int n0 = slice * 16 * kLmQ4MaxNB;
  const int v_wave = slab * kSlab + wave * kRows;
  const int G = p.H / 64;
  const int words = p.H / 8;

  // code words of this lane's rows (clamped into range; rows past V are ignored)
  const uint32_t* wrow[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
    wrow[vb] = p.wq + static_cast<int64_t>(min(v_wave + 16 * vb + li, p.V - 1)) * words + 2 * lg;
  // (scale, bias) of the lane's output rows 16 vb + 4 lg .. +3 (V % 4 == 0,
  // so the four pairs are one aligned 16-byte load; clamped rows stay in range)
  int srow[VB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) srow[vb] = min(v_wave + 16 * vb + 4 * lg, p.V - 4);
  auto sb_load = [&](int vb, int c) {
    return *reinterpret_cast<const u32x4*>(p.sb + 2 * (static_cast<int64_t>(c) * p.V + srow[vb]));
  };
  // the four scales of a (scale, bias) load as two bf16 pairs; its four
  // biases go to the wave's LDS rows (the 16 lanes of a lane group hold the
  // same rows: one of them writes)
  auto scales = [](u32x4 sb) -> u32x2 {
    return u32x2{__builtin_amdgcn_perm(sb[1], sb[0], 0x05040100u), __builtin_amdgcn_perm(sb[3], sb[2], 0x05040100u)};
  };
  auto keep_biases = [&](int vb, u32x4 sb, int g) {
    if (li == 0)
      *reinterpret_cast<u32x2*>(&s_bias[wave][g & 63][16 * vb + 4 * lg]) =
          u32x2{__builtin_amdgcn_perm(sb[1], sb[0], 0x07060302u), __builtin_amdgcn_perm(sb[3], sb[2], 0x07060302u)};
  };
  // hidden-state staging: piece t covers row t / 8, bytes 16 (t % 8) of the group
  constexpr int kPieces = 16 * NB * 8;
  constexpr int kPiecesPerThread = (kPieces + kLmQ4Threads - 1) / kLmQ4Threads;
  auto x_piece = [&](int c, int r) -> u32x4 {
    const int t = threadIdx.x + kLmQ4Threads * r;
    const int row = min(n0 + t / 8, p.N - 1);
    const unsigned char* src = reinterpret_cast<const unsigned char*>(p.x + static_cast<int64_t>(row) * p.x_stride) +
                               c * (kLmKc * 2) + 16 * (t % 8);
    return *reinterpret_cast<const u32x4*>(src);
  };
  auto x_store = [&](int buf, int r, u32x4 v) {
    const int t = threadIdx.x + kLmQ4Threads * r;
    *reinterpret_cast<u32x4*>(&s_x[buf][(t / 8) * kLmXPitch + 16 * (t % 8)]) = v;
  };

  f32x4 acc[VB][NB];
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[vb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Stages the group sums of the chunk starting at g0 (groups g0 .. g0 + 31
  // of the padded planes, in bounds) into s_xg with direct global -> LDS
  // loads, no registers: load j of the workgroup fills slots 64 j .. +63,
  // slot q being row q / 5, 16-byte part q % 5. The pad part of a row and any
  // slot past the rows load a valid address and are never read.
  auto stage_xg = [&](int g0) {
    const uint32_t base = lds_u32(s_xg);
    for (int j = wave; j < kXgDma; j += NW) {
      const int q = 64 * j + lane;
      const int row = min(q / (kXgPitch / 16), kXgRows - 1);
      const int part = min(q % (kXgPitch / 16), 3);
      const int sp = row / (16 * NB), n = min(n0 + row % (16 * NB), p.N - 1);
      dma16v_at(p.xg + (static_cast<size_t>(sp) * p.N + n) * p.Gp + g0 + 8 * part, base + 1024 * j);
    }
  };
  // acc += bias (rows x groups) . X (groups x nodes) over groups g0 .. g0 + 31
  // (those past G are zero): A = the wave's biases (lane (i, g) holds row i,
  // groups g0 + 8 g .. + 7), B = X as its three bf16 terms (lane (i, g) holds
  // node i's groups g0 + 8 g .. + 7)
  auto bias_chunk = [&](int g0) {
    bf16x8 bf[VB];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      uint32_t bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int g = g0 + 8 * lg + e;
        const uint32_t b = s_bias[wave][g & 63][16 * vb + li];
        bv[e] = g < G ? b : 0u;
      }
      bf[vb] = __builtin_bit_cast(bf16x8, u32x4{bv[0] | (bv[1] << 16), bv[2] | (bv[3] << 16), bv[4] | (bv[5] << 16),
                                                bv[6] | (bv[7] << 16)});
    }
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 xb = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&s_xg[(sp * 16 * NB + 16 * nb + li) * kXgPitch + 16 * lg]));
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
          acc[vb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[vb], xb, acc[vb][nb], 0, 0, 0);
      }
  };

  u32x4 xs[kPiecesPerThread];
#pragma unroll
  for (int r = 0; r < kPiecesPerThread; ++r)
    if (threadIdx.x + kLmQ4Threads * r < kPieces) xs[r] = x_piece(0, r);
#pragma unroll
  for (int r = 0; r < kPiecesPerThread; ++r)
    if (threadIdx.x + kLmQ4Threads * r < kPieces) x_store(0, r, xs[r]);
  // Code words and (scale, bias) pairs two groups ahead, in a two-slot
  // register ring: slot c & 1 holds group c's, and is refilled with group
  // c + 2's right after group c has been converted, so no loaded register is
  // copied from one step to the next (a copy of a register still loading
  // would wait for that load, exposing its latency every step). The group
  // loop is unrolled by two so that the slot index is known at compile time.
  // Issue order per step: the next group's hidden pieces, then group c + 2's
  // words and pairs; the step ends waiting for its hidden pieces, which (the
  // load counter completes in issue order) also covers what the step before
  // issued, but nothing issued after the pieces.
  const int last = G - 1;
  u32x2 wr[2][VB];
  u32x4 sbw[2][VB];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      wr[q][vb] = *reinterpret_cast<const u32x2*>(wrow[vb] + 8 * min(q, last));
      sbw[q][vb] = sb_load(vb, min(q, last));
    }
  __syncthreads();

  auto step = [&](int c, auto slot_tag) __attribute__((always_inline)) {
    constexpr int Q = decltype(slot_tag)::value;  // == c & 1
    const int buf = Q;
    const bool more = c + 1 < G;
    // the last step of a chunk of 32 groups (or of the row) stages the
    // chunk's group sums for its bias product, ahead of the step's loads
    const bool chunk_end = (c & 31) == 31 || c == last;
    if (chunk_end) stage_xg(c & ~31);
    if (more) {
#pragma unroll
      for (int r = 0; r < kPiecesPerThread; ++r)
        if (threadIdx.x + kLmQ4Threads * r < kPieces) xs[r] = x_piece(c + 1, r);
    }
    // the group's codes as bf16 (both 32-element halves), its scales, and
    // its biases into this wave's LDS rows
    bf16x8 wf[VB][2];
    float sc[VB][4];
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) wf[vb][h] = __builtin_bit_cast(bf16x8, q4_to_bf16x8(wr[Q][vb][h]));
      const u32x2 scw = scales(sbw[Q][vb]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = scw[j >> 1];
        sc[vb][j] = __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
      }
      keep_biases(vb, sbw[Q][vb], c);
    }
    // refill the slot with group c + 2 (past the end: a re-read of the last
    // group, never used)
    const int c2 = min(c + 2, last);
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      wr[Q][vb] = *reinterpret_cast<const u32x2*>(wrow[vb] + 8 * c2);
      sbw[Q][vb] = sb_load(vb, c2);
    }

    // One node block at a time: the group's partial sums of block nb (two
    // MFMAs from zero), and in their shadow the fold of block nb - 1 into the
    // running logits, acc += scale * partial (output row 16 vb + 4 lg + j,
    // node 16 nb + li). Only two blocks of partial sums are live.
    auto fold = [&](const f32x4 (&part)[VB], int nb) __attribute__((always_inline)) {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[vb][nb][j] = fmaf(sc[vb][j], part[vb][j], acc[vb][nb][j]);
          // ties the fold to this point of the schedule (emits nothing):
          // otherwise the folds, used only by the next group, sink below the
          // scheduling barriers to the end of the group
          asm volatile("" : "+v"(acc[vb][nb][j]));
        }
    };
    // block nb + 1's hidden fragments are read while block nb multiplies; a
    // scheduling barrier closes each block, so the compiler cannot gather the
    // MFMAs of all blocks first and leave the folds to the end
    auto x_frag = [&](int nb, int h) {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(&s_x[buf][(16 * nb + li) * kLmXPitch + 32 * lg + 16 * h]));
    };
    f32x4 prev[VB];
    bf16x8 x0 = x_frag(0, 0), x1 = x_frag(0, 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bf16x8 y0 = x0, y1 = x1;
      if (nb + 1 < NB) {
        y0 = x_frag(nb + 1, 0);
        y1 = x_frag(nb + 1, 1);
      }
      f32x4 cur[VB];
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        cur[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[vb][0], x0, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        cur[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[vb][1], x1, cur[vb], 0, 0, 0);
      }
      if (nb > 0) fold(prev, nb - 1);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) prev[vb] = cur[vb];
      x0 = y0;
      x1 = y1;
      __builtin_amdgcn_sched_barrier(0);
    }
    fold(prev, NB - 1);
    if (more) {
#pragma unroll
      for (int r = 0; r < kPiecesPerThread; ++r)
        if (threadIdx.x + kLmQ4Threads * r < kPieces) x_store(buf ^ 1, r, xs[r]);
    }
    // the staging loads came before the step's 2 VB refill loads: once at
    // most that many are outstanding, they have landed (in issue order)
    if (chunk_end) wait_vmcnt<2 * VB>();
    __syncthreads();
    // a finished chunk: its bias product (its biases were kept by this wave;
    // its group sums are staged)
    if (chunk_end) bias_chunk(c & ~31);
  };
  int c = 0;
  for (; c + 1 < G; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    step(c + 1, std::integral_constant<int, 1>{});
  }
  if (c < G) step(c, std::integral_constant<int, 0>{});

  // epilogue: node 16 nb + li's best over the lane's rows 16 vb + 4 lg + j
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    uint64_t best = 0;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = v_wave + 16 * vb + 4 * lg + j;
        if (v < p.V) {
          const uint64_t k = lm_key(acc[vb][nb][j], static_cast<uint32_t>(v));
          best = k > best ? k : best;
        }
      }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const uint64_t o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
    if (lg == 0) s_best[wave][16 * nb + li] = best;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 16 * NB && n0 + t < p.N) {
    uint64_t best = s_best[0][t];
#pragma unroll
    for (int w = 1; w < NW; ++w) best = s_best[w][t] > best ? s_best[w][t] : best;
    p.part[static_cast<int64_t>(n0 + t) * p.n_slabs + slab] = best;
  }
}

// one wave per node: the best key over the vocabulary slabs
__global__ void __launch_bounds__(kWave) lm_head_reduce(const uint64_t* __restrict__ part, int n_slabs,
                                                        int32_t* __restrict__ out_idx) {
  const int n = blockIdx.x;
  const uint64_t* __restrict__ r = part + static_cast<int64_t>(n) * n_slabs;
  uint64_t best = 0;
  for (int s = threadIdx.x; s < n_slabs; s += kWave) best = r[s] > best ? r[s] : best;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if (threadIdx.x == 0) out_idx[n] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best));
}

// row blocks per wave for a call of n_rows nodes (the node blocks of its
// first slice decide), and the vocabulary slabs of kLmWaves such waves
static int lm_vb(int64_t n_rows) { return n_rows > 16 * (kLmMaxNB - 1) ? 2 : kLmMaxVB; }
static int lm_slabs(int64_t n_rows, int64_t vocab) {
  const int64_t rows = int64_t{kLmWaves} * 16 * lm_vb(n_rows);
  return static_cast<int>((vocab + rows - 1) / rows);
}

}  // namespace ttv

using namespace ttv;

extern "C" size_t lm_head_argmax_ws(int64_t n_rows, int64_t vocab) {
  if (n_rows <= 0 || vocab <= 0) return 0;
  return static_cast<size_t>(n_rows) * lm_slabs(n_rows, vocab) * sizeof(uint64_t);
}

extern "C" ttv_status lm_head_argmax(const uint16_t* hidden, int64_t n_rows, int64_t hidden_stride,
                                     const uint16_t* weight, int64_t vocab, int64_t hidden_dim, int64_t weight_stride,
                                     int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(n_rows >= 0 && n_rows <= (1 << 24), TTV_ERR_INVALID, "lm_head_argmax: n_rows %lld not in [0, 2^24]",
              (long long)n_rows);
  if (n_rows == 0) return TTV_OK;
  TTV_REQUIRE(vocab >= 1 && vocab <= 0x7FFFFFFF, TTV_ERR_INVALID, "lm_head_argmax: vocab %lld not in [1, 2^31 - 1]",
              (long long)vocab);
  TTV_REQUIRE(hidden_dim >= kLmKc && hidden_dim % kLmKc == 0 && hidden_dim <= (1 << 20), TTV_ERR_INVALID,
              "lm_head_argmax: hidden_dim %lld is not a positive multiple of %d (<= 2^20)", (long long)hidden_dim,
              kLmKc);
  TTV_REQUIRE(hidden_stride >= hidden_dim && hidden_stride % 8 == 0 && weight_stride >= hidden_dim &&
                  weight_stride % 8 == 0,
              TTV_ERR_INVALID, "lm_head_argmax: strides (%lld, %lld) must be >= hidden_dim and multiples of 8",
              (long long)hidden_stride, (long long)weight_stride);
  TTV_REQUIRE(hidden && weight && out_idx, TTV_ERR_INVALID, "lm_head_argmax: NULL pointer");
  TTV_REQUIRE(reinterpret_cast<uintptr_t>(hidden) % 16 == 0 && reinterpret_cast<uintptr_t>(weight) % 16 == 0,
              TTV_ERR_INVALID, "lm_head_argmax: hidden and weight must be 16-byte aligned");
  const size_t need = lm_head_argmax_ws(n_rows, vocab);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "lm_head_argmax: workspace %zu bytes < %zu", ws_bytes, need);
  LmParams p;
  p.x = hidden;
  p.w = weight;
  p.part = static_cast<uint64_t*>(ws);
  p.x_stride = hidden_stride;
  p.w_stride = weight_stride;
  p.N = static_cast<int>(n_rows);
  p.V = static_cast<int>(vocab);
  p.H = static_cast<int>(hidden_dim);
  p.n_slabs = lm_slabs(n_rows, vocab);
  p.n_slices = static_cast<int>((n_rows + 16 * kLmMaxNB - 1) / (16 * kLmMaxNB));
  const int64_t n_wg = static_cast<int64_t>(p.n_slabs) * p.n_slices;
  TTV_REQUIRE(n_wg <= (1ll << 30), TTV_ERR_INVALID, "lm_head_argmax: too many workgroups");
  const unsigned grid = static_cast<unsigned>((n_wg + kNumXcd - 1) / kNumXcd * kNumXcd);
  // node blocks per slice: enough for the nodes of the (first) slice
  const int rows0 = static_cast<int>(n_rows < 16 * kLmMaxNB ? n_rows : 16 * kLmMaxNB);
  const int nb = (rows0 + 15) / 16;
  hipStream_t s = (hipStream_t)stream;
  switch (nb) {
#define TTV_LM(NB) \
  case NB: hipLaunchKernelGGL((lm_head_main<NB, NB == kLmMaxNB ? 2 : kLmMaxVB>), dim3(grid), dim3(kLmThreads), 0, s, p); break;
    TTV_LM(1) TTV_LM(2) TTV_LM(3) TTV_LM(4) TTV_LM(5) TTV_LM(6) TTV_LM(7) TTV_LM(8)
#undef TTV_LM
    default: return fail(TTV_ERR_INVALID, "lm_head_argmax: internal node-block count");
  }
  ttv_status st = check_launch("lm_head_argmax main");
  if (st != TTV_OK) return st;
  hipLaunchKernelGGL(lm_head_reduce, dim3(static_cast<unsigned>(n_rows)), dim3(kWave), 0, s,
                     static_cast<const uint64_t*>(p.part), p.n_slabs, out_idx);
  return check_launch("lm_head_argmax reduce");
}

// workspace: the best key per (node, slab), then the group sums' three bf16
// planes [3][n_rows][Gp] (256-byte aligned)
static size_t lm_q4_part_bytes(int64_t n_rows, int64_t vocab) {
  const size_t b = static_cast<size_t>(n_rows) * static_cast<size_t>((vocab + kLmQ4Slab - 1) / kLmQ4Slab) *
                   sizeof(uint64_t);
  return (b + 255) / 256 * 256;
}
static int lm_q4_gp(int64_t hidden_dim) { return static_cast<int>((hidden_dim / 64 + 31) / 32 * 32); }

extern "C" size_t lm_head_q4_argmax_ws(int64_t n_rows, int64_t vocab, int64_t hidden_dim) {
  if (n_rows <= 0 || vocab <= 0 || hidden_dim < 64) return 0;
  return lm_q4_part_bytes(n_rows, vocab) + 3 * static_cast<size_t>(n_rows) * lm_q4_gp(hidden_dim) * sizeof(uint16_t);
}

extern "C" ttv_status lm_head_q4_argmax(const uint16_t* hidden, int64_t n_rows, int64_t hidden_stride,
                                        const uint32_t* wq, const uint16_t* scale_bias, int64_t vocab,
                                        int64_t hidden_dim, int32_t* out_idx, void* ws, size_t ws_bytes,
                                        void* stream) {
  clear_error();
  TTV_REQUIRE(n_rows >= 0 && n_rows <= (1 << 24), TTV_ERR_INVALID,
              "lm_head_q4_argmax: n_rows %lld not in [0, 2^24]", (long long)n_rows);
  if (n_rows == 0) return TTV_OK;
  TTV_REQUIRE(vocab >= 4 && vocab % 4 == 0 && vocab <= 0x7FFFFFFF, TTV_ERR_INVALID,
              "lm_head_q4_argmax: vocab %lld must be a multiple of 4 in [4, 2^31 - 1]", (long long)vocab);
  TTV_REQUIRE(hidden_dim >= 64 && hidden_dim % 64 == 0 && hidden_dim <= (1 << 20), TTV_ERR_INVALID,
              "lm_head_q4_argmax: hidden_dim %lld is not a positive multiple of 64 (<= 2^20)",
              (long long)hidden_dim);
  TTV_REQUIRE(hidden_stride >= hidden_dim && hidden_stride % 8 == 0, TTV_ERR_INVALID,
              "lm_head_q4_argmax: hidden_stride %lld must be >= hidden_dim and a multiple of 8",
              (long long)hidden_stride);
  TTV_REQUIRE(hidden && wq && scale_bias && out_idx, TTV_ERR_INVALID, "lm_head_q4_argmax: NULL pointer");
  TTV_REQUIRE(reinterpret_cast<uintptr_t>(hidden) % 16 == 0 && reinterpret_cast<uintptr_t>(wq) % 8 == 0 &&
                  reinterpret_cast<uintptr_t>(scale_bias) % 16 == 0,
              TTV_ERR_INVALID, "lm_head_q4_argmax: hidden and scale_bias must be 16-byte aligned, wq 8-byte");
  TTV_REQUIRE(vocab * (hidden_dim / 8) <= (int64_t{1} << 40), TTV_ERR_INVALID, "lm_head_q4_argmax: head too large");
  const size_t need = lm_head_q4_argmax_ws(n_rows, vocab, hidden_dim);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "lm_head_q4_argmax: workspace %zu bytes < %zu", ws_bytes,
              need);
  LmQ4Params p;
  p.x = hidden;
  p.wq = wq;
  p.sb = scale_bias;
  p.part = static_cast<uint64_t*>(ws);
  p.xg = reinterpret_cast<const uint16_t*>(static_cast<char*>(ws) + lm_q4_part_bytes(n_rows, vocab));
  p.x_stride = hidden_stride;
  p.N = static_cast<int>(n_rows);
  p.V = static_cast<int>(vocab);
  p.H = static_cast<int>(hidden_dim);
  p.Gp = lm_q4_gp(hidden_dim);
  const int rows0 = static_cast<int>(n_rows < 16 * kLmQ4MaxNB ? n_rows : 16 * kLmQ4MaxNB);
  const int nb = (rows0 + 15) / 16;
  p.n_slabs = static_cast<int>((vocab + kLmQ4Slab - 1) / kLmQ4Slab);
  p.n_slices = static_cast<int>((n_rows + 16 * kLmQ4MaxNB - 1) / (16 * kLmQ4MaxNB));
  const int64_t n_wg = static_cast<int64_t>(p.n_slabs) * p.n_slices;
  TTV_REQUIRE(n_wg <= (1ll << 30), TTV_ERR_INVALID, "lm_head_q4_argmax: too many workgroups");
  const int64_t n_sums = n_rows * p.Gp;
  TTV_REQUIRE(n_sums <= (int64_t{1} << 36), TTV_ERR_INVALID, "lm_head_q4_argmax: too many group sums");
  hipStream_t s = (hipStream_t)stream;
  {
    hipLaunchKernelGGL(lm_q4_group_sums, dim3(static_cast<unsigned>((n_sums + 255) / 256)), dim3(256), 0, s, hidden,
                       hidden_stride, p.N, p.H / 64, p.Gp, const_cast<uint16_t*>(p.xg));
    ttv_status st = check_launch("lm_head_q4_argmax group sums");
    if (st != TTV_OK) return st;
  }
  const unsigned grid = static_cast<unsigned>((n_wg + kNumXcd - 1) / kNumXcd * kNumXcd);
  switch (nb) {
#define TTV_LMQ(NB, NW, VB) \
  case NB: hipLaunchKernelGGL((lm_head_q4_main<NB, NW, VB>), dim3(grid), dim3(NW * kWave), 0, s, p); break;
    TTV_LMQ(1, 8, 2) TTV_LMQ(2, 8, 2) TTV_LMQ(3, 8, 2) TTV_LMQ(4, 8, 2)
    TTV_LMQ(5, 8, 2) TTV_LMQ(6, 8, 2) TTV_LMQ(7, 8, 2) TTV_LMQ(8, 8, 2)
#undef TTV_LMQ
    default: return fail(TTV_ERR_INVALID, "lm_head_q4_argmax: internal node-block count");
  }
  ttv_status st = check_launch("lm_head_q4_argmax main");
  if (st != TTV_OK) return st;
  hipLaunchKernelGGL(lm_head_reduce, dim3(static_cast<unsigned>(n_rows)), dim3(kWave), 0, s,
                     static_cast<const uint64_t*>(p.part), p.n_slabs, out_idx);
  return check_launch("lm_head_q4_argmax reduce");
}
