// Step 2 of a verify round: tree-masked GQA verify attention.
//
// [I1204] mlxcel issue #1204, "Redirection": attention verifies a tree by
// flattening its nodes into one sequence and handing the forward the tree
// mask, so siblings cannot see each other. [PR1212] mlxcel PR #1212,
// history-mask commit: every node attends the whole cached history and, inside
// the block, its ancestors and itself; the block's rows sit at P + i in node
// order (rollback-to-path commit). Gemma 4 tree-verify commit: a linear tree
// must reproduce the linear path bit for bit -- here the causal case (anc ==
// NULL) is literally the linear tree's bitset, so both run the same code.
//
// Work decomposition (one wavefront per workgroup):
//   unit  = (sequence b, KV head g, row chunk rc). The rows of a unit are the
//           (node, query head) pairs of the G query heads sharing KV head g:
//           row r = node * G + head-in-group. Every K/V byte of the unit is
//           read once for all of its rows (GQA sharing).
//   split = a range of split_len prefix keys; the last split of a unit also
//           takes the block keys [P, P + T) under the ancestor bitsets.
//   Each workgroup keeps an online softmax (running max m, sum l, unnormalised
//   output) over its keys. With one split it writes the output directly;
//   otherwise it stores (m, l, o) partials and the last workgroup of the unit
//   to finish (device-scope counter) merges them by log-sum-exp. Workgroups
//   are laid out XCD-contiguously so a unit's splits share one L2.
//
// MFMA path (bf16 queries, bf16 or int8 KV, D = 128, >= 16 rows): 32-key tiles
// stream straight from HBM into registers -- no LDS. With lane = (i = lane %
// 16, g = lane / 16) and v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T : A = K (16 keys x 32 d), B = Q^T (32 d x 16 rows). The two
//       16-key blocks of a tile take keys 8(i/4) + 4kb + i%4, so the output
//       lane (i, g) receives keys 8g .. 8g+7 of query row i.
//   O^T = V^T P^T (v_mfma_f32_16x16x32_f16): B = P^T is exactly that lane's
//       8 probabilities (k-slot group g <-> keys 8g..8g+7), rounded to fp16.
//       A = V^T with output row m of d-block db standing for d = 8m + db, so
//       lane (i, g) needs V[8g + e][8i .. 8i+8) for e = 0..7: eight contiguous
//       16-byte (bf16) or 8-byte (int8) loads, regrouped in registers. No
//       transpose through LDS is needed.
//   Precision: bf16 values and int8 codes convert to fp16 exactly, so the only
//       rounding in P V is the fp16 probability (2^-12 relative); a bf16
//       probability (2^-9) would not hold a 2e-3 bound once a short prefix
//       makes the softmax peaked. bf16 V must therefore lie in fp16 range.
//   int8 KV: codes (|c| <= 127) convert exactly to bf16/fp16; the per-token
//       scales fold into the scores (s = (q . c) * k_scale) and into the
//       probabilities (p' = p * v_scale), so the matrix cores only see codes.
// VALU path (fp32 everything, or fewer than 16 rows): one key per lane for
// scores, one d per lane for the output, queries and probabilities in LDS.
#include "common.hpp"

namespace ttv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMfmaMaxRB = 4;   // row blocks of 16 per MFMA workgroup (64 rows)
constexpr int kValuRows = 16;   // rows per VALU workgroup
constexpr int kTargetWG = 1024;
constexpr int kMaxSplits = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const uint16_t* ks;
  const uint16_t* vs;
  const uint64_t* anc;
  float* out;
  float* part_o;
  float* part_ml;
  int32_t* counters;
  int B, Hq, Hkv, G, D, cap, split_len, rows_chunk, nwg;
  float scale_log2;
  int32_t node_off[TTV_MAX_BATCH + 1];
  int32_t hist_len[TTV_MAX_BATCH];
  int32_t wg_off[TTV_MAX_BATCH + 1];
  int32_t unit_off[TTV_MAX_BATCH + 1];
};

struct Work {
  int b, kvh, split, rc, nsplit, rc_n, P, T, o0, rows, row0, nrows, unit, slot, k_lo, k_hi;
  bool last;
};

__device__ __forceinline__ void decode(const AttnParams& p, int slot, Work& w) {
  int lo = 0, hi = p.B;  // wg_off[lo] <= slot < wg_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.wg_off[mid] <= slot) lo = mid; else hi = mid;
  }
  w.b = lo;
  w.o0 = p.node_off[lo];
  w.T = p.node_off[lo + 1] - w.o0;
  w.P = p.hist_len[lo];
  w.rows = w.T * p.G;
  w.rc_n = (w.rows + p.rows_chunk - 1) / p.rows_chunk;
  w.nsplit = w.P > 0 ? (w.P + p.split_len - 1) / p.split_len : 1;
  int rem = slot - p.wg_off[lo];
  w.rc = rem % w.rc_n;
  rem /= w.rc_n;
  w.split = rem % w.nsplit;
  w.kvh = rem / w.nsplit;
  w.unit = p.unit_off[lo] + w.kvh * w.rc_n + w.rc;
  w.slot = slot;
  w.row0 = w.rc * p.rows_chunk;
  w.nrows = min(p.rows_chunk, w.rows - w.row0);
  w.k_lo = w.split * p.split_len;
  w.k_hi = min(w.P, w.k_lo + p.split_len);
  w.last = w.split == w.nsplit - 1;
}

// Ancestor bitset of a row's node; NULL anc is the linear (causal) tree, whose
// node t sees block nodes 0..t.
__device__ __forceinline__ uint64_t row_bits(const AttnParams& p, const Work& w, int row) {
  const int t = row / p.G;
  if (p.anc) return p.anc[w.o0 + t];
  return (2ull << t) - 1ull;  // t = 63 wraps to all ones
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Merge of a unit's split partials by log-sum-exp; run by the last workgroup
// of the unit. Partials: o [slot][rows_chunk][D], (m, l) [slot][rows_chunk][2].
__device__ void merge_unit(const AttnParams& p, const Work& w) {
  const int lane = threadIdx.x;
  const int slot0 = p.wg_off[w.b] + (w.kvh * w.nsplit) * w.rc_n + w.rc;
  const int step = w.rc_n;
  for (int r = 0; r < w.nrows; ++r) {
    float M = -INFINITY;
    for (int s = 0; s < w.nsplit; ++s) M = fmaxf(M, p.part_ml[((size_t)(slot0 + s * step) * p.rows_chunk + r) * 2]);
    float L = 0.f;
    float acc0 = 0.f, acc1 = 0.f;
    for (int s = 0; s < w.nsplit; ++s) {
      const size_t pr = (size_t)(slot0 + s * step) * p.rows_chunk + r;
      const float ms = p.part_ml[pr * 2];
      const float ls = p.part_ml[pr * 2 + 1];
      const float wt = ms == -INFINITY ? 0.f : exp2f(ms - M);
      L += wt * ls;
      const float* po = p.part_o + pr * p.D;
      acc0 += wt * po[lane];
      if (p.D == 128) acc1 += wt * po[lane + 64];
    }
    const int row = w.row0 + r;
    const int node = w.o0 + row / p.G;
    const int qh = w.kvh * p.G + row % p.G;
    float* o = p.out + ((size_t)node * p.Hq + qh) * p.D;
    const float inv = 1.0f / L;
    o[lane] = acc0 * inv;
    if (p.D == 128) o[lane + 64] = acc1 * inv;
  }
}

// After a split has written its partials: count it; the last one merges.
__device__ __forceinline__ void finish_split(const AttnParams& p, const Work& w) {
  __threadfence();
  int last = 0;
  if (threadIdx.x == 0) last = atomicAdd(&p.counters[w.unit], 1) == w.nsplit - 1;
  last = __shfl(last, 0);
  if (!last) return;
  __threadfence();
  merge_unit(p, w);
  if (threadIdx.x == 0) atomicExch(&p.counters[w.unit], 0);
}

// ------------------------------------------------------------- MFMA path ----

__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(lo >> (8 * k))));
    r[4 + k] = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(hi >> (8 * k))));
  }
  return r;
}

template <bool I8, int RB>
__global__ void __launch_bounds__(64) attn_mfma_kernel(const AttnParams p) {
  const int slot = xcd_slot(blockIdx.x, p.nwg);
  if (slot < 0) return;
  Work w;
  decode(p, slot, w);
  const int lane = threadIdx.x;
  const int li = lane & 15;
  const int lg = lane >> 4;
  constexpr int D = 128;

  // Q^T fragments, staged once in LDS in lane order (one conflict-free 16-byte
  // read per fragment per tile). k-slot mapping of the QK product (shared by K
  // and Q): bf16 KV d = 32ks + 8g + e; int8 KV d = 32g + 8ks + e (so a lane's
  // 32 int8 codes are contiguous).
  __shared__ u32x4 qs[RB][4][64];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rloc = rb * 16 + li;
    const bool ok = rloc < w.nrows;
    const int row = w.row0 + (ok ? rloc : 0);
    const int node = w.o0 + row / p.G;
    const int qh = w.kvh * p.G + row % p.G;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)node * p.Hq + qh) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d0 = I8 ? 32 * lg + 8 * ks : 32 * ks + 8 * lg;
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (!ok) x = u32x4{0, 0, 0, 0};
      qs[rb][ks][lane] = x;
    }
  }
  __syncthreads();

  f32x4 o[8][RB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t head = (size_t)w.b * p.Hkv + w.kvh;
  const char* kbase = static_cast<const char*>(p.k) + head * p.cap * D * (I8 ? 1 : 2);
  const char* vbase = static_cast<const char*>(p.v) + head * p.cap * D * (I8 ? 1 : 2);
  const uint16_t* ksb = I8 ? p.ks + head * p.cap : nullptr;
  const uint16_t* vsb = I8 ? p.vs + head * p.cap : nullptr;
  constexpr int RBYTES = I8 ? D : 2 * D;

  // mode 0: full prefix tile; 1: prefix tile ending at `limit`; 2: block tile
  // (tbits: ancestor bitsets of the lane's rows, used in mode 2 only)
  auto tile = [&](int t0, int mode, int limit, const uint64_t* tbits) {
    // ---- loads (indices clamped to limit - 1 in boundary tiles) ----
    bf16x8 kf[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int key = t0 + 8 * (li >> 2) + 4 * kb + (li & 3);
      if (mode != 0) key = min(key, limit - 1);
      const char* kr = kbase + (size_t)key * RBYTES;
      if constexpr (I8) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * lg));
        const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * lg + 16));
        kf[kb][0] = i8x8_to_bf16(a[0], a[1]);
        kf[kb][1] = i8x8_to_bf16(a[2], a[3]);
        kf[kb][2] = i8x8_to_bf16(c[0], c[1]);
        kf[kb][3] = i8x8_to_bf16(c[2], c[3]);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kf[kb][ks] = __builtin_bit_cast(
              bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 2 * (32 * ks + 8 * lg))));
      }
    }
    u32x4 vr[8];
    u32x2 vr8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int key = t0 + 8 * lg + e;
      if (mode != 0) key = min(key, limit - 1);
      const char* vrow = vbase + (size_t)key * RBYTES;
      if constexpr (I8)
        vr8[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vrow + 8 * li));
      else
        vr[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vrow + 16 * li));
    }
    float fk[8], fv[8];
    if constexpr (I8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int key = t0 + 8 * lg + e;
        if (mode != 0) key = min(key, limit - 1);
        fk[e] = fp16_to_f32(ksb[key]) * p.scale_log2;
        fv[e] = fp16_to_f32(vsb[key]);
      }
    }

    // ---- S^T = K Q^T ----
    f32x4 sacc[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 qf = __builtin_bit_cast(bf16x8, qs[rb][ks][lane]);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf, a1, 0, 0, 0);
      }
      sacc[0][rb] = a0;
      sacc[1][rb] = a1;
    }

    // ---- online softmax; lane holds keys 8g + e of row i ----
    // Lazy rescaling: a row's reference max m only moves when the tile max
    // exceeds it by more than 2^6 (any lane -> the whole wave takes the
    // rescale branch), so probabilities stay below 64 (p * v_scale stays in
    // fp16 range for any fp16 scale) and the accumulators are rescaled a
    // handful of times per workgroup instead of every tile.
    f16x8 pt[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = sacc[e >> 2][rb][e & 3];
        x[e] = I8 ? s * fk[e] : s * p.scale_log2;
        if (mode == 1) {
          if (t0 + 8 * lg + e >= limit) x[e] = -INFINITY;
        } else if (mode == 2) {
          const int kt = t0 - w.P + 8 * lg + e;
          if (t0 + 8 * lg + e >= limit || !((tbits[rb] >> kt) & 1ull)) x[e] = -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (__ballot(mx > m[rb] + 6.0f) != 0) {
        const float mnew = fmaxf(m[rb], mx);
        const float alpha = mnew == -INFINITY ? 1.0f : exp2f(m[rb] - mnew);
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
        m[rb] = mnew;
      }
      const float msub = m[rb] == -INFINITY ? 0.f : m[rb];
      float sum = 0.f;
      f16x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pe = exp2f(x[e] - msub);
        sum += pe;
        if constexpr (I8) pe *= fv[e];
        pv[e] = static_cast<_Float16>(pe);
      }
      l[rb] += sum;
      pt[rb] = pv;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      f16x8 vf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float f;
        if constexpr (I8) {
          f = static_cast<float>(static_cast<int8_t>(vr8[e][db >> 2] >> (8 * (db & 3))));
        } else {
          const uint32_t wv = vr[e][db >> 1];
          f = __uint_as_float((db & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
        }
        vf[e] = static_cast<_Float16>(f);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pt[rb], o[db][rb], 0, 0, 0);
    }
  };

  int t0 = w.k_lo;
#pragma nounroll
  for (; t0 + 32 <= w.k_hi; t0 += 32) tile(t0, 0, 0, nullptr);
  if (t0 < w.k_hi) tile(t0, 1, w.k_hi, nullptr);
  if (w.last) {
    uint64_t bits[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rloc = rb * 16 + li;
      bits[rb] = rloc < w.nrows ? row_bits(p, w, w.row0 + rloc) : 1ull;
    }
#pragma nounroll
    for (int tt = 0; tt < w.T; tt += 32) tile(w.P + tt, 2, w.P + w.T, bits);
  }

  // ---- epilogue ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l[rb] += __shfl_xor(l[rb], 16);
    l[rb] += __shfl_xor(l[rb], 32);
  }
  const bool direct = w.nsplit == 1;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rloc = rb * 16 + li;
    if (rloc >= w.nrows) continue;
    float* dst;
    float scl;
    if (direct) {
      const int row = w.row0 + rloc;
      const int node = w.o0 + row / p.G;
      const int qh = w.kvh * p.G + row % p.G;
      dst = p.out + ((size_t)node * p.Hq + qh) * D;
      scl = 1.0f / l[rb];
    } else {
      const size_t pr = (size_t)w.slot * p.rows_chunk + rloc;
      dst = p.part_o + pr * D;
      scl = 1.0f;
      if (lg == 0) {
        p.part_ml[pr * 2] = m[rb];
        p.part_ml[pr * 2 + 1] = l[rb];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 v = {o[4 * h][rb][r], o[4 * h + 1][rb][r], o[4 * h + 2][rb][r], o[4 * h + 3][rb][r]};
        *reinterpret_cast<f32x4*>(dst + 32 * lg + 8 * r + 4 * h) = v * scl;
      }
  }
  if (!direct) finish_split(p, w);
}

// ------------------------------------------------------------- VALU path ----

template <int KT>
__device__ __forceinline__ void load8(const void* base, size_t idx, float* f) {
  if constexpr (KT == TTV_F32) {
    const f32x4* q = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    const f32x4 a = q[0], b = q[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  } else if constexpr (KT == TTV_BF16) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(a[e] << 16);
      f[2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
    }
  } else {
    const u32x2 a = *reinterpret_cast<const u32x2*>(static_cast<const int8_t*>(base) + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = static_cast<float>(static_cast<int8_t>(a[0] >> (8 * e)));
      f[4 + e] = static_cast<float>(static_cast<int8_t>(a[1] >> (8 * e)));
    }
  }
}

template <int KT>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  if constexpr (KT == TTV_F32) return static_cast<const float*>(base)[idx];
  else if constexpr (KT == TTV_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return static_cast<float>(static_cast<const int8_t*>(base)[idx]);
}

template <int QT, int KT, int D>
__global__ void __launch_bounds__(64) attn_valu_kernel(const AttnParams p) {
  constexpr int R = kValuRows;
  constexpr int C = D / 64;
  __shared__ float qs[R][D];
  __shared__ f32x4 ps[64][R / 4];
  const int slot = xcd_slot(blockIdx.x, p.nwg);
  if (slot < 0) return;
  Work w;
  decode(p, slot, w);
  const int lane = threadIdx.x;
  for (int idx = lane; idx < R * D; idx += 64) {
    const int r = idx / D, d = idx % D;
    float val = 0.f;
    if (r < w.nrows) {
      const int row = w.row0 + r;
      const int node = w.o0 + row / p.G;
      const int qh = w.kvh * p.G + row % p.G;
      const size_t qi = ((size_t)node * p.Hq + qh) * D + d;
      val = QT == TTV_F32 ? static_cast<const float*>(p.q)[qi] : bf16_to_f32(static_cast<const uint16_t*>(p.q)[qi]);
    }
    qs[r][d] = val;
  }
  __syncthreads();
  const size_t head = (size_t)w.b * p.Hkv + w.kvh;
  const size_t kv0 = head * p.cap;
  float m[R], l[R], o[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) o[r][c] = 0.f;
  }
  uint64_t bits[R];
#pragma unroll
  for (int r = 0; r < R; ++r) bits[r] = ~0ull;

  auto tile = [&](int t0, int mode, int limit) {
    const int key = t0 + lane;
    const bool valid = mode == 0 || key < limit;
    const int kk = valid ? key : limit - 1;
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 8) {
      float kv[8];
      load8<KT>(p.k, (kv0 + kk) * D + d0, kv);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[r] = fmaf(qs[r][d0 + e], kv[e], s[r]);
    }
    float fk = p.scale_log2, fv = 1.f;
    if constexpr (KT == TTV_I8) {
      fk *= fp16_to_f32(p.ks[kv0 + kk]);
      fv = fp16_to_f32(p.vs[kv0 + kk]);
    }
    float pr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float x = s[r] * fk;
      if (!valid || (mode == 2 && !((bits[r] >> (key - w.P)) & 1ull))) x = -INFINITY;
      const float mnew = fmaxf(m[r], wave_max(x));
      const float msub = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(m[r] - msub);
      const float pe = exp2f(x - msub);
      l[r] = l[r] * alpha + wave_sum(pe);
      m[r] = mnew;
#pragma unroll
      for (int c = 0; c < C; ++c) o[r][c] *= alpha;
      pr[r] = pe * fv;
    }
#pragma unroll
    for (int r4 = 0; r4 < R / 4; ++r4) ps[lane][r4] = f32x4{pr[4 * r4], pr[4 * r4 + 1], pr[4 * r4 + 2], pr[4 * r4 + 3]};
    __syncthreads();
    const int nk = mode == 0 ? 64 : min(64, limit - t0);
    for (int j = 0; j < nk; ++j) {
      float vv[C];
#pragma unroll
      for (int c = 0; c < C; ++c) vv[c] = load1<KT>(p.v, (kv0 + t0 + j) * D + lane + 64 * c);
#pragma unroll
      for (int r4 = 0; r4 < R / 4; ++r4) {
        const f32x4 pj = ps[j][r4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < C; ++c) o[4 * r4 + u][c] = fmaf(pj[u], vv[c], o[4 * r4 + u][c]);
      }
    }
    __syncthreads();
  };

  int t0 = w.k_lo;
  for (; t0 + 64 <= w.k_hi; t0 += 64) tile(t0, 0, 0);
  if (t0 < w.k_hi) tile(t0, 1, w.k_hi);
  if (w.last) {
#pragma unroll
    for (int r = 0; r < R; ++r) bits[r] = r < w.nrows ? row_bits(p, w, w.row0 + r) : 1ull;
    tile(w.P, 2, w.P + w.T);  // T <= 64: one tile
  }

  const bool direct = w.nsplit == 1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= w.nrows) continue;
    float* dst;
    float scl;
    if (direct) {
      const int row = w.row0 + r;
      const int node = w.o0 + row / p.G;
      const int qh = w.kvh * p.G + row % p.G;
      dst = p.out + ((size_t)node * p.Hq + qh) * D;
      scl = 1.0f / l[r];
    } else {
      const size_t pr = (size_t)w.slot * p.rows_chunk + r;
      dst = p.part_o + pr * D;
      scl = 1.0f;
      if (lane == 0) {
        p.part_ml[pr * 2] = m[r];
        p.part_ml[pr * 2 + 1] = l[r];
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) dst[lane + 64 * c] = o[r][c] * scl;
  }
  if (!direct) finish_split(p, w);
}

// ------------------------------------------------------------- planning ----

struct AttnPlan {
  bool mfma;
  int rb;
  AttnParams prm;  // everything except pointers
  int nunits;
  size_t off_ml, off_o, ws_bytes;
};

static ttv_status plan_attention(const ttv_batch* batch, int Hq, const ttv_kv_layer* L, int q_dtype,
                                 AttnPlan& pl) {
  ttv_status s = check_batch(batch, false);
  if (s != TTV_OK) return s;
  TTV_REQUIRE(L != nullptr, TTV_ERR_INVALID, "tree_verify_attention: layer is NULL");
  TTV_REQUIRE(L->Hkv > 0 && Hq > 0 && Hq % L->Hkv == 0, TTV_ERR_INVALID,
              "tree_verify_attention: Hq %d is not a multiple of Hkv %d", Hq, L->Hkv);
  TTV_REQUIRE(L->D == 64 || L->D == 128, TTV_ERR_INVALID, "tree_verify_attention: head_dim %d not in {64, 128}",
              L->D);
  const bool f32 = q_dtype == TTV_F32 && L->dtype == TTV_F32;
  const bool bf = q_dtype == TTV_BF16 && (L->dtype == TTV_BF16 || L->dtype == TTV_I8);
  TTV_REQUIRE(f32 || bf, TTV_ERR_UNSUPPORTED,
              "tree_verify_attention: unsupported q/KV dtype pair (%d, %d); supported: f32/f32, bf16/bf16, bf16/i8",
              q_dtype, L->dtype);
  if (L->dtype == TTV_I8)
    TTV_REQUIRE(L->k_scale && L->v_scale, TTV_ERR_UNSUPPORTED,
                "tree_verify_attention: int8 KV needs its fp16 scale sidecars");
  const int B = batch->B;
  const int G = Hq / L->Hkv;
  int max_rows = 0, maxP = 0;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    const int P = batch->hist_len_h[b];
    TTV_REQUIRE((int64_t)P + T <= L->cap, TTV_ERR_INVALID,
                "tree_verify_attention: sequence %d needs P + T = %d rows, cache holds %d", b, P + T, L->cap);
    max_rows = T * G > max_rows ? T * G : max_rows;
    maxP = P > maxP ? P : maxP;
  }
  pl.mfma = bf && L->D == 128 && max_rows >= 16;
  if (pl.mfma) {
    // balanced row chunks of at most 64 rows: e.g. 80 rows -> 2 x 48
    const int nch = (max_rows + 16 * kMfmaMaxRB - 1) / (16 * kMfmaMaxRB);
    const int per = (max_rows + nch - 1) / nch;
    pl.rb = (per + 15) / 16;
  } else {
    pl.rb = 0;
  }
  AttnParams& p = pl.prm;
  p = AttnParams{};
  p.B = B;
  p.Hq = Hq;
  p.Hkv = L->Hkv;
  p.G = G;
  p.D = L->D;
  p.cap = L->cap;
  p.rows_chunk = pl.mfma ? 16 * pl.rb : kValuRows;
  int64_t work = 0;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    const int rc = (T * G + p.rows_chunk - 1) / p.rows_chunk;
    const int P = batch->hist_len_h[b];
    work += (int64_t)p.Hkv * rc * (P > 0 ? P : 1);
  }
  int64_t sl = (work + kTargetWG - 1) / kTargetWG;
  const int64_t min_sl = (maxP + kMaxSplits - 1) / kMaxSplits;
  if (sl < min_sl) sl = min_sl;
  if (sl < 256) sl = 256;
  sl = (sl + 63) / 64 * 64;
  p.split_len = static_cast<int>(sl);
  int wg = 0, units = 0;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    const int P = batch->hist_len_h[b];
    const int rc = (T * G + p.rows_chunk - 1) / p.rows_chunk;
    const int ns = P > 0 ? (P + p.split_len - 1) / p.split_len : 1;
    p.node_off[b] = batch->node_off_h[b];
    p.hist_len[b] = P;
    p.wg_off[b] = wg;
    p.unit_off[b] = units;
    wg += p.Hkv * ns * rc;
    units += p.Hkv * rc;
  }
  p.node_off[B] = batch->node_off_h[B];
  p.wg_off[B] = wg;
  p.unit_off[B] = units;
  p.nwg = wg;
  pl.nunits = units;
  const size_t counters = ((size_t)units * 4 + 255) / 256 * 256;
  pl.off_ml = counters;
  pl.off_o = pl.off_ml + ((size_t)wg * p.rows_chunk * 2 * 4 + 255) / 256 * 256;
  pl.ws_bytes = pl.off_o + (size_t)wg * p.rows_chunk * p.D * 4;
  return TTV_OK;
}

}  // namespace ttv

using namespace ttv;

extern "C" size_t tree_verify_attention_ws(const ttv_batch* batch, int32_t Hq, const ttv_kv_layer* layer,
                                           int32_t q_dtype) {
  AttnPlan pl;
  if (plan_attention(batch, Hq, layer, q_dtype, pl) != TTV_OK) return 0;
  return pl.ws_bytes;
}

extern "C" ttv_status tree_verify_attention(const ttv_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                                            const ttv_kv_layer* layer, const uint64_t* anc, float softmax_scale,
                                            float* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  AttnPlan pl;
  ttv_status s = plan_attention(batch, Hq, layer, q_dtype, pl);
  if (s != TTV_OK) return s;
  if (pl.prm.nwg == 0) return TTV_OK;
  TTV_REQUIRE(q && out && layer->k && layer->v, TTV_ERR_INVALID, "tree_verify_attention: NULL pointer");
  TTV_REQUIRE(ws && ws_bytes >= pl.ws_bytes, TTV_ERR_WORKSPACE,
              "tree_verify_attention: workspace %zu bytes < %zu", ws_bytes, pl.ws_bytes);
  AttnParams p = pl.prm;
  p.q = q;
  p.k = layer->k;
  p.v = layer->v;
  p.ks = layer->dtype == TTV_I8 ? layer->k_scale : nullptr;
  p.vs = layer->dtype == TTV_I8 ? layer->v_scale : nullptr;
  p.anc = anc;
  p.out = out;
  p.counters = static_cast<int32_t*>(ws);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_ml);
  p.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_o);
  p.scale_log2 = softmax_scale * kLog2e;
  const unsigned grid = static_cast<unsigned>((p.nwg + kNumXcd - 1) / kNumXcd * kNumXcd);
  hipStream_t st = (hipStream_t)stream;
  const bool i8 = layer->dtype == TTV_I8;
  if (pl.mfma) {
#define TTV_MFMA(I, R) hipLaunchKernelGGL((attn_mfma_kernel<I, R>), dim3(grid), dim3(64), 0, st, p)
    switch (pl.rb) {
      case 1: if (i8) TTV_MFMA(true, 1); else TTV_MFMA(false, 1); break;
      case 2: if (i8) TTV_MFMA(true, 2); else TTV_MFMA(false, 2); break;
      case 3: if (i8) TTV_MFMA(true, 3); else TTV_MFMA(false, 3); break;
      default: if (i8) TTV_MFMA(true, 4); else TTV_MFMA(false, 4); break;
    }
#undef TTV_MFMA
  } else {
#define TTV_VALU(Q, K, DD) hipLaunchKernelGGL((attn_valu_kernel<Q, K, DD>), dim3(grid), dim3(64), 0, st, p)
    if (q_dtype == TTV_F32) {
      if (p.D == 64) TTV_VALU(TTV_F32, TTV_F32, 64); else TTV_VALU(TTV_F32, TTV_F32, 128);
    } else if (!i8) {
      if (p.D == 64) TTV_VALU(TTV_BF16, TTV_BF16, 64); else TTV_VALU(TTV_BF16, TTV_BF16, 128);
    } else {
      if (p.D == 64) TTV_VALU(TTV_BF16, TTV_I8, 64); else TTV_VALU(TTV_BF16, TTV_I8, 128);
    }
#undef TTV_VALU
  }
  return check_launch("tree_verify_attention");
}
