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
// Work decomposition:
//   unit  = (sequence b, KV head g, row chunk rc). The rows of a unit are the
//           (node, query head) pairs of the G query heads sharing KV head g:
//           row r = node * G + head-in-group. Every K/V byte of the unit is
//           read once for all of its rows (GQA sharing).
//   split = a range of split_len prefix keys; the last split of a unit also
//           takes the block keys [P, P + T) under the ancestor bitsets.
//   Each split keeps its softmax against a per-row reference m (set from its
//   first tile), the row sums l and the unnormalised output over its keys. A unit covered by one workgroup is written
//   directly; otherwise every workgroup stores one (m, l, o) partial and a
//   second launch merges a unit's partials by log-sum-exp.
//
// MFMA path (bf16 queries, bf16 or int8 KV, D = 128; a block of fewer than 16
// rows is padded with zero queries): workgroups of 4 wave pairs, the two
// waves of a pair on one SIMD, K/V streamed through LDS in 32-key tiles by
// LDS-DMA. Three kernels:
//   attn_i8_split_kernel   int8 KV. The pairs take 4 consecutive splits of
//                          one unit (XCD-contiguous workgroups); a pair's
//                          score wave forms S and the probabilities, its
//                          value wave accumulates O and issues every load.
//   attn_bf16_narrow_kernel bf16 KV, at most 96 rows per KV head. The pairs
//                          take 4 consecutive splits; the two waves of a pair
//                          split the rows and stage half of every tile each.
//   attn_bf16_split_kernel bf16 KV, more rows. The pairs take up to 4 row
//                          chunks of one (KV head, split) and share one ring;
//                          split by phase as the int8 kernel. Workgroups are
//                          dealt round-robin to the XCDs, longest first.
// With lane = (i = lane % 16, g = lane / 16) and
// v_mfma_f32_16x16x32_{bf16,f16}:
//   S^T = K Q^T : A = K (16 keys x 32 d), B = Q^T (32 d x 16 rows). The two
//       16-key blocks of a tile take keys 8(i/4) + 4kb + i%4, so the output
//       lane (i, g) receives keys 8g .. 8g+7 of query row i.
//   O^T = V^T P^T (v_mfma_f32_16x16x32_f16): B = P^T is exactly that lane's
//       8 probabilities (k-slot group g <-> keys 8g..8g+7), rounded to fp16.
//       A = V^T, lane (i, g) holding V[8g + e][d] for e = 0..7 of its d.
//   Precision: bf16 values (in fp16 range) and int8 codes convert to fp16
//       exactly, so the only rounding in P V is the fp16 probability (2^-12
//       relative); a bf16 probability (2^-9) would not hold a 2e-3 bound once
//       a short prefix makes the softmax peaked. bf16 V must therefore lie in
//       fp16 range.
//   int8 KV: codes (|c| <= 127) convert exactly to fp16; the per-token scales
//       fold into the scores (s = (q . c) * k_scale) and into the
//       probabilities (p' = p * v_scale), so the matrix cores only see codes.
// VALU path (fp32 queries and KV, D = 64, caches of fewer than 32 rows, and
// windows the MFMA kernels do not take): one key per lane for scores, one d
// per lane for the output, queries and probabilities in LDS.
#include "common.hpp"

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

namespace ttv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

constexpr int kMfmaMaxRB = 6;   // row blocks of 16 per MFMA row chunk (96 rows, two waves)
constexpr int kI8MaxRB = 5;     // int8: both waves of a pair hold all row blocks (80 rows)
constexpr int kValuRows = 16;   // rows per VALU workgroup
constexpr int kTargetWG = 1024;
constexpr int kWideTargetWG = 512;
constexpr int kWideMaxRB = 5;  // bf16 wide layout: row blocks per row chunk (one pair of waves each)
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
  int32_t* exact_flags;  // int8 path: per workgroup, 1 = its rows take the exact code conversion
  int B, Hq, Hkv, G, D, cap, split_len, rows_chunk, nwg, split_pad;
  int wide;  // wide layout: the row chunks of one (kv head, split) take ceil(rc_n / 4) * 4 consecutive slots
  int window;  // sliding-window layers: node i (cache row P + i) keeps keys > P + i - window; 0 = none
  float scale_log2;
  int32_t node_off[TTV_MAX_BATCH + 1];
  int32_t hist_len[TTV_MAX_BATCH];
  int32_t wg_off[TTV_MAX_BATCH + 1];
  int32_t unit_off[TTV_MAX_BATCH + 1];
  int32_t rchunk[TTV_MAX_BATCH];  // rows per chunk of sequence b (<= rows_chunk, the partials' row stride)
  // wide layout, dispatch order: every workgroup of a full-length split first
  // (sequence by sequence), then the workgroups of each sequence's last split,
  // longest first. full_off[b]: full-split workgroups of sequences before b;
  // last_key[k] = (last-split workgroups of the k longest before k) << 8 | b
  int32_t full_off[TTV_MAX_BATCH + 1];
  int32_t last_key[TTV_MAX_BATCH + 1];
};
static_assert(sizeof(AttnParams) <= 4096, "kernel arguments");

struct Work {
  int b, kvh, split, rc, nsplit, rc_n, P, T, o0, rows, row0, nrows, unit, slot, k_lo, k_hi;
  bool last;
};

// First history key any row of a sequence can see: with a window, node 0
// (row P) keeps keys > P - window, so history keys below P - window + 1 are
// read by no row and the unit's splits start there.
__host__ __device__ __forceinline__ int hist_key_start(int P, int window) {
  return (window > 0 && P - window + 1 > 0) ? P - window + 1 : 0;
}

// Splits of sequence b (the same count decode() derives).
__host__ __device__ __forceinline__ int seq_splits(const AttnParams& p, int b) {
  const int P = p.hist_len[b];
  const int ks = hist_key_start(P, p.window);
  const int ns = P > ks ? (P - ks + p.split_len - 1) / p.split_len : 1;
  return (ns + p.split_pad - 1) / p.split_pad * p.split_pad;
}

// Wide layout: the workgroup that dispatch position g runs. Every workgroup
// of a full-length split comes first, the short last splits after them,
// longest first, so the last workgroups to start are the shortest ones.
// Workgroup index wgi = wg_off[b] / 4 + (kvh * nsplit + split) * grp + group,
// grp = the sequence's groups of four row chunks.
__device__ __forceinline__ int wide_order(const AttnParams& p, int g) {
  int b, kvh, split, grp_i;
  const int nfull = p.full_off[p.B];
  auto groups = [&](int bb) {
    const int rows = (p.node_off[bb + 1] - p.node_off[bb]) * p.G;
    const int rc = (rows + p.rchunk[bb] - 1) / p.rchunk[bb];
    return (rc + 3) / 4;
  };
  if (g < nfull) {
    int lo = 0, hi = p.B;  // full_off[lo] <= g < full_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.full_off[mid] <= g) lo = mid; else hi = mid;
    }
    b = lo;
    const int grp = groups(b), ns = seq_splits(p, b);
    const int idx = g - p.full_off[b];
    kvh = idx / ((ns - 1) * grp);
    const int r = idx % ((ns - 1) * grp);
    split = r / grp;
    grp_i = r % grp;
  } else {
    const int g2 = g - nfull;
    int lo = 0, hi = p.B;  // (last_key[lo] >> 8) <= g2 < (last_key[hi] >> 8)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((p.last_key[mid] >> 8) <= g2) lo = mid; else hi = mid;
    }
    b = p.last_key[lo] & 255;
    const int grp = groups(b);
    const int idx = g2 - (p.last_key[lo] >> 8);
    kvh = idx / grp;
    grp_i = idx % grp;
    split = seq_splits(p, b) - 1;
  }
  return p.wg_off[b] / 4 + (kvh * seq_splits(p, b) + split) * groups(b) + grp_i;
}

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
  const int rch = p.rchunk[lo];
  w.rc_n = (w.rows + rch - 1) / rch;
  const int ks = hist_key_start(w.P, p.window);
  const int ns = w.P > ks ? (w.P - ks + p.split_len - 1) / p.split_len : 1;
  w.nsplit = (ns + p.split_pad - 1) / p.split_pad * p.split_pad;  // trailing splits may be empty
  int rem = slot - p.wg_off[lo];
  if (p.wide) {  // the row chunks of one (kv head, split) are consecutive slots
    const int rcg = (w.rc_n + 3) / 4 * 4;
    w.rc = rem % rcg;
    rem /= rcg;
    w.split = rem % w.nsplit;
    w.kvh = rem / w.nsplit;
  } else {
    w.split = rem % w.nsplit;
    rem /= w.nsplit;
    w.rc = rem % w.rc_n;
    w.kvh = rem / w.rc_n;
  }
  w.unit = p.unit_off[lo] + w.kvh * w.rc_n + w.rc;
  w.slot = slot;
  w.row0 = w.rc * rch;
  w.nrows = max(0, min(rch, w.rows - w.row0));  // 0: a padding chunk of the wide layout
  w.k_lo = ks + w.split * p.split_len;
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

// The key tiles of a work item, in processing order: prefix tiles over
// [k_lo, k_hi) (the last may be partial), then on the last split the block
// tiles over [P, P + T). Under a sliding window node i keeps keys
// j >= P - window + 1 + i (key j > P + i - window), so the first keys of the
// unit's range are seen by some rows and not by others; the tiles holding
// them ("edge" tiles, at most two: T <= 64) go behind the other prefix tiles
// and are masked per row, so that the first tile, whose scores set the rows'
// references, is one that every row sees whole. Tile modes: 0 a full prefix
// tile, 1 the partial last prefix tile, 2 a block tile (ancestor bits),
// 3 an edge tile (keys >= edge_lo + the row's node).
struct TileList {
  int k_lo, k_hi, P, T, edge_lo, n_edge, n_rest, n_pref, n_full, ntile;
  __device__ __forceinline__ void init(const AttnParams& p, const Work& w, int kt) {
    k_lo = w.k_lo;
    k_hi = w.k_hi;
    P = w.P;
    T = w.T;
    edge_lo = P - p.window + 1;
    const int edge_end = min(edge_lo + T - 1, k_hi);  // keys below it are hidden from some row
    n_edge = p.window > 0 && edge_end > k_lo ? (edge_end - k_lo + kt - 1) / kt : 0;
    const int rest_lo = k_lo + kt * n_edge;
    n_rest = k_hi > rest_lo ? (k_hi - rest_lo + kt - 1) / kt : 0;
    n_full = k_hi > rest_lo ? (k_hi - rest_lo) / kt : 0;  // the leading mode-0 tiles
    n_pref = n_edge + n_rest;
    ntile = n_pref + (w.last ? (T + kt - 1) / kt : 0);
  }
  __device__ __forceinline__ void geom(int t, int kt, int& t0, int& mode, int& limit) const {
    if (t < n_rest) {
      t0 = k_lo + kt * (n_edge + t);
      limit = k_hi;
      mode = t0 + kt <= k_hi ? 0 : 1;
    } else if (t < n_pref) {
      t0 = k_lo + kt * (t - n_rest);
      limit = k_hi;
      mode = 3;
    } else {
      t0 = P + kt * (t - n_pref);
      limit = P + T;
      mode = 2;
    }
    t0 = __builtin_amdgcn_readfirstlane(t0);
  }
};

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

// Merge of n partials of one unit by log-sum-exp, by the whole workgroup of
// kMergeThreads, over rows [r0, r1) of the unit's chunk (r1 - r0 <=
// kMergeRows). Partials: o [slot][rows_chunk][D] and (m, l)
// [slot][rows_chunk][2] for slots slot0 + s * stride, s < n <= kMaxSplits
// (m = -inf marks an empty split). First the weights: the 8 lanes of row r
// take partials j, j + 8, ... of it, and with M = max m_s and
// L = sum 2^(m_s - M) l_s write w_s = 2^(m_s - M) / L into wt (LDS, by the
// row's place in [r0, r1)); then out = sum_s w_s o_s, every thread with the
// loads of 8 partials of its output in flight at once.
constexpr int kMergeRows = 16;                     // rows per merge workgroup (grid y)
constexpr int kMergeThreads = 8 * kMergeRows;      // 8 lanes per row for the weights
constexpr int kMergeWt = kMergeRows * kMaxSplits;  // weights of one merge workgroup, at most
static_assert(kMergeWt * sizeof(float) <= 8192, "merge weight table");
__device__ void merge_partials(const AttnParams& p, const Work& w, int slot0, int n, float* wt, int r0, int r1,
                               int stride) {
  const int tid = threadIdx.x;
  {
    const int r = r0 + (tid >> 3), j = tid & 7;
    const bool live = r < r1;
    constexpr int C = kMaxSplits / 8;
    float ms[C], ls[C];
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int sidx = j + 8 * c;
      ms[c] = -INFINITY;
      ls[c] = 0.f;
      if (live && sidx < n) {
        const size_t pr = (size_t)(slot0 + sidx * stride) * p.rows_chunk + r;
        ms[c] = p.part_ml[pr * 2];
        ls[c] = p.part_ml[pr * 2 + 1];
      }
      M = fmaxf(M, ms[c]);
    }
    M = fmaxf(M, __shfl_xor(M, 1));
    M = fmaxf(M, __shfl_xor(M, 2));
    M = fmaxf(M, __shfl_xor(M, 4));
    float L = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      ms[c] = ms[c] == -INFINITY ? 0.f : exp2f(ms[c] - M);  // the weight, before 1 / L
      L += ms[c] * ls[c];
    }
    L += __shfl_xor(L, 1);
    L += __shfl_xor(L, 2);
    L += __shfl_xor(L, 4);
    const float inv = 1.0f / L;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (live && j + 8 * c < n) wt[(r - r0) * kMaxSplits + j + 8 * c] = ms[c] * inv;
  }
  __syncthreads();
  const int D4 = p.D / 4;
  for (int idx = tid; idx < (r1 - r0) * D4; idx += kMergeThreads) {
    const int rl = idx / D4, d4 = idx % D4;
    const int r = r0 + rl;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += 8) {
      f32x4 os[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        os[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s0 + k < n)
          os[k] = reinterpret_cast<const f32x4*>(p.part_o + ((size_t)(slot0 + (s0 + k) * stride) * p.rows_chunk + r) *
                                                 p.D)[d4];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < n) acc += wt[rl * kMaxSplits + s0 + k] * os[k];
    }
    const int row = w.row0 + r;
    const int node = w.o0 + row / p.G;
    const int qh = w.kvh * p.G + row % p.G;
    reinterpret_cast<f32x4*>(p.out + ((size_t)node * p.Hq + qh) * p.D)[d4] = acc;
  }
}

// Second launch: one workgroup per (unit, block of kMergeRows rows) of the
// units whose keys were split over more than one partial merges them (a kernel boundary orders the partials' stores
// before these loads; an in-kernel device-scope fence would write back whole
// L2 caches). per_slot: key splits per stored partial (4 for the MFMA path,
// whose workgroups fold their 4 splits first; 1 for the VALU path).
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const AttnParams p, int per_slot) {
  __shared__ float wt[kMergeWt];
  const int u = blockIdx.x;
  int lo = 0, hi = p.B;  // unit_off[lo] <= u < unit_off[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.unit_off[mid] <= u) lo = mid; else hi = mid;
  }
  Work w;
  w.b = lo;
  w.o0 = p.node_off[lo];
  w.T = p.node_off[lo + 1] - w.o0;
  w.P = p.hist_len[lo];
  w.rows = w.T * p.G;
  const int rch = p.rchunk[lo];
  w.rc_n = (w.rows + rch - 1) / rch;
  const int ks = hist_key_start(w.P, p.window);
  const int ns = w.P > ks ? (w.P - ks + p.split_len - 1) / p.split_len : 1;
  w.nsplit = (ns + p.split_pad - 1) / p.split_pad * p.split_pad;
  const int n = w.nsplit / per_slot;
  if (u >= p.unit_off[lo + 1] || n <= 1) return;
  const int rem = u - p.unit_off[lo];
  w.kvh = rem / w.rc_n;
  w.rc = rem % w.rc_n;
  w.row0 = w.rc * rch;
  w.nrows = min(rch, w.rows - w.row0);
  const int r0 = blockIdx.y * kMergeRows;
  if (r0 >= w.nrows) return;
  const int rcg = (w.rc_n + 3) / 4 * 4;
  if (p.wide)  // split s of this chunk is slot group (kvh, s), member rc
    merge_partials(p, w, p.wg_off[lo] + w.kvh * w.nsplit * rcg + w.rc, n, wt, r0, min(w.nrows, r0 + kMergeRows),
                   rcg);
  else
    merge_partials(p, w, (p.wg_off[lo] + rem * w.nsplit) / per_slot, n, wt, r0, min(w.nrows, r0 + kMergeRows), 1);
}

// ------------------------------------------------------------- MFMA path ----

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// int8 code -> fp16, exactly: with u = c ^ 0x80 = c + 128 (as an unsigned byte)
// the fp16 bit pattern 0x64uu is 1024 + u, and 1024 + u - 1152 = c. v_perm
// places two bytes under the 0x64 exponent bytes, one packed f16 add removes
// the offset.
constexpr uint32_t kExp64 = 0x64646464u;
__device__ __forceinline__ uint32_t f16pair_from_bytes(uint32_t sel_src, uint32_t sel) {
  const f16x2 off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kExp64, sel_src, sel)) + off);
}
// The same bytes as fp16 of c + 1152, exactly, in one v_perm per pair: the
// MFMA paths that can take the constant offset back out of their results
// (a start value of the accumulator, a row sum) skip the packed add.
constexpr float kCodeBias = 1152.0f;
__device__ __forceinline__ f16x8 i8x8_to_f16_biased(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(kExp64, lo, 0x04010400u);
  r[1] = __builtin_amdgcn_perm(kExp64, lo, 0x04030402u);
  r[2] = __builtin_amdgcn_perm(kExp64, hi, 0x04010400u);
  r[3] = __builtin_amdgcn_perm(kExp64, hi, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}
// 8 int8 codes (two dwords, already xor-ed with 0x80808080) -> 8 fp16
__device__ __forceinline__ f16x8 i8x8_to_f16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = f16pair_from_bytes(lo, 0x04010400u);
  r[1] = f16pair_from_bytes(lo, 0x04030402u);
  r[2] = f16pair_from_bytes(hi, 0x04010400u);
  r[3] = f16pair_from_bytes(hi, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}

// Wait until this wave's LDS reads (and scalar loads) have returned.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __asm__ volatile("" ::: "memory");
}

// Wait until at most `ahead` tiles of ND DMAs each are outstanding (ahead <= 5).
template <int ND>
__device__ __forceinline__ void wait_vmcnt_tiles(int ahead) {
  if (ahead >= 5) wait_vmcnt<5 * ND>();
  else if (ahead == 4) wait_vmcnt<4 * ND>();
  else if (ahead == 3) wait_vmcnt<3 * ND>();
  else if (ahead == 2) wait_vmcnt<2 * ND>();
  else if (ahead == 1) wait_vmcnt<ND>();
  else wait_vmcnt<0>();
}

// LDS layout of a staged K or V tile: 32 rows of RBYTES, 16-byte chunks. The
// logical chunk c of row r sits at physical chunk c ^ swz(r), chosen so that
// the 16 rows one fragment read touches (rows 8a + 4kb + b) land in 16
// different bank groups; for int8 tiles also the 8 rows 8g .. 8g + 7 that one
// transposed V read touches (a 128-byte row is half a bank row, so even and
// odd rows take the two halves and the swizzle keeps each half's rows apart).
template <bool I8>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (I8) return ((r >> 1) & 3) ^ (((r >> 3) & 1) << 1) ^ (((r >> 4) & 1) << 2);  // 8 chunks per row
  else return ((r >> 3) & 3) | ((r & 3) << 2);                                            // 16 chunks per row
}

__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, const void* lds) {
  dma16_at(sbase, voff, lds_u32(lds));
}
__device__ __forceinline__ void dma16v(const void* g, const void* lds) { dma16v_at(g, lds_u32(lds)); }

// A workgroup is NP = 4 wave pairs: the pairs take 4 consecutive key splits
// of one unit, and the two waves of a pair split the unit's row chunk (RB0
// row blocks of 16 rows, then RB1) and share one LDS ring, each staging half
// of every tile. 512 threads at 2 waves per SIMD: 256 registers per wave.
// (bf16 KV with at most 96 rows per KV head; int8 KV and wider bf16 chunks
// take the kernels split by phase below.)
template <int RB0, int RB1, int S>
__global__ void __launch_bounds__(512) attn_bf16_narrow_kernel(const AttnParams p) {
  constexpr int NP = 4;                       // wave pairs = consecutive key splits
  constexpr int NW = 2 * NP;                  // waves
  constexpr int RBU = RB0 + RB1;              // row blocks of the unit's row chunk
  constexpr int D = 128;
  constexpr int RBYTES = 2 * D;               // bytes of one K (or V) row
  constexpr int CH = RBYTES / 16;             // 16-byte chunks per row
  constexpr int KT = 32;                      // keys per tile
  constexpr int KBYTES = KT * RBYTES;         // one K (or V) tile
  constexpr int NK = KBYTES / 1024;           // DMA instructions per K (or V) tile
  constexpr int TILE = 2 * KBYTES;            // K tile, then V tile
  // per pair: an S-stage ring of K/V tiles; per workgroup: the unit's Q^T
  // fragments (one conflict-free 16-byte read per use) and ancestor bitsets
  __shared__ __attribute__((aligned(16))) char ring_all[NP][S][TILE];
  __shared__ __attribute__((aligned(16))) u32x4 qsh[RBU * 4 * 64];
  __shared__ uint64_t tbits_s[RBU * 16];
  __shared__ int s_nt[NP];

  const int wgi = xcd_slot(blockIdx.x, p.nwg / NP);
  if (wgi < 0) return;  // whole workgroup
  // The wave index as a uniform value: the wave's whole work item then lives in
  // scalar registers and every branch on it is a scalar branch.
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int pair = wave & (NP - 1);  // the pair's two waves sit on one SIMD
  const int h = wave / NP;  // 0: row blocks [0, RB0), stages K; 1: [RB0, RBU), stages V
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;
  Work w;
  decode(p, wgi * NP + pair, w);  // the pairs share (b, kv head, row chunk)
  char (*ring)[TILE] = ring_all[pair];

  // Q^T fragments into LDS. k-slot mapping of the QK product (shared by K and
  // Q): d = 32ks + 8g + e.
  for (int f = wave; f < RBU * 4; f += NW) {
    const int rb = f >> 2, ks = f & 3;
    const int rloc = rb * 16 + li;
    const bool ok = rloc < w.nrows;
    const int row = ok ? w.row0 + rloc : 0;
    const int node = w.o0 + row / p.G;
    const int qh = w.kvh * p.G + row % p.G;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)node * p.Hq + qh) * D;
    u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
    if (!ok) x = u32x4{0, 0, 0, 0};
    qsh[f * 64 + lane] = x;
  }
  // ancestor bitsets of the unit's rows, needed by block tiles only
  for (int r = threadIdx.x; r < RBU * 16; r += 64 * NW)
    tbits_s[r] = r < w.nrows ? row_bits(p, w, w.row0 + r) : 1ull;
  // every ordinary load has landed before the DMA ring starts, so the waits in
  // the loop count ring traffic only
  wait_vmcnt<0>();
  __syncthreads();

  const size_t head = (size_t)w.b * p.Hkv + w.kvh;
  const char* kbase = static_cast<const char*>(p.k) + head * p.cap * RBYTES;
  const char* vbase = static_cast<const char*>(p.v) + head * p.cap * RBYTES;

  // Per-lane DMA geometry: piece j of a K (or V) tile is tile row
  // r = (64 j + lane) / CH, 16-byte chunk (64 j + lane) % CH of that row
  // (swizzled), i.e. byte koff[j] of the tile.
  auto piece_row = [&](int j) { return (64 * j + lane) / CH; };
  auto piece_col = [&](int j) {
    return 16u * static_cast<uint32_t>(((64 * j + lane) % CH) ^ lds_swz<false>(piece_row(j)));
  };
  uint32_t koff[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) koff[j] = static_cast<uint32_t>(piece_row(j) * RBYTES) + piece_col(j);

  // Tile list (full prefix tiles first, then the partial, edge and block ones)
  TileList tl;
  tl.init(p, w, KT);
  const int ntile = tl.ntile;
  const int n_full = tl.n_full;
  auto geom = [&](int t, int& t0, int& mode, int& limit) { tl.geom(t, KT, t0, mode, limit); };

  // DMA this wave's half of one tile into ring slot t % S: the K half or the
  // V half, exactly NK instructions. Full
  // tiles use the precomputed offsets; boundary tiles clamp every row into
  // [t0, limit) so they stay in bounds.
  const char* hbase = h == 0 ? kbase : vbase;
  auto issue = [&](int t) {
    int t0, mode, limit;
    geom(t, t0, mode, limit);
    char* dst = ring[t % S] + (h == 0 ? 0 : KBYTES);
    const char* src = hbase + (size_t)t0 * RBYTES;
    if (mode == 0) {
#pragma unroll
      for (int j = 0; j < NK; ++j) dma16(src, koff[j], dst + 1024 * j);
    } else {
      const int lim = limit - 1 - t0;
#pragma unroll
      for (int j = 0; j < NK; ++j)
        dma16(src, static_cast<uint32_t>(min(piece_row(j), lim) * RBYTES) + piece_col(j), dst + 1024 * j);
    }
  };
  // this wave's half of tile t has landed: at most its halves of the tiles
  // issued after t are still outstanding
  auto wait_tile = [&](int t) {
    wait_vmcnt_tiles<NK>(min(S - 2, ntile - 1 - t));
  };

  // The pair's two waves each stage half of every tile, so a tile is complete
  // once both halves landed: one workgroup barrier per tile. It also frees the
  // slot of the previous tile for the next DMA. All waves run the workgroup's
  // longest tile list (the last split also takes the block tiles).
#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < ntile) issue(t);
  if (lane == 0 && h == 0) s_nt[pair] = ntile;
  if (ntile > 0) wait_tile(0);
  __syncthreads();
  int nt_wg = 0;
#pragma unroll
  for (int q = 0; q < NP; ++q) nt_wg = max(nt_wg, s_nt[q]);
  // the fold goes through LDS, in the rings' space
  float* mo = reinterpret_cast<float*>(&ring_all[0][0][0]);
  float* mml = mo + RBU * 32 * 64;  // mo: [RBU][8][4][64] lane-major o; mml: [RBU * 16][2] (m, l)
  static_assert(RBU * 32 * 64 * 4 + RBU * 16 * 8 <= NP * S * TILE, "fold area");
  // Row-major stores of rows [0, wq.nrows) of a chunk from mo / mml, four
  // consecutive d per thread (coalesced): the unit's output if one partial
  // covers it, else partial slot `slot`. LDS holds o in the MFMA lane order:
  // row 16 rb + i, d = 32 g + 8 r + db at ((rb * 8 + db) * 4 + r) * 64 + 16 g + i.
  auto store_out = [&](const Work& wq, int slot, bool whole) {
    for (int flat = 4 * threadIdx.x; flat < wq.nrows * D; flat += 4 * 64 * NW) {
      const int rloc = flat / D, d0 = flat % D;
      const int rb = rloc >> 4, i = rloc & 15;
      f32x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = d0 + u;
        v[u] = mo[((rb * 8 + (d & 7)) * 4 + ((d >> 3) & 3)) * 64 + 16 * (d >> 5) + i];
      }
      if (whole) {
        const int row = wq.row0 + rloc;
        const int node = wq.o0 + row / p.G;
        const int qh = wq.kvh * p.G + row % p.G;
        *reinterpret_cast<f32x4*>(p.out + ((size_t)node * p.Hq + qh) * D + d0) = v / mml[rloc * 2 + 1];
      } else {
        *reinterpret_cast<f32x4*>(p.part_o + ((size_t)slot * p.rows_chunk + rloc) * D + d0) = v;
      }
    }
    if (!whole) {
      for (int r = threadIdx.x; r < wq.nrows; r += 64 * NW) {
        p.part_ml[((size_t)slot * p.rows_chunk + r) * 2] = mml[r * 2];
        p.part_ml[((size_t)slot * p.rows_chunk + r) * 2 + 1] = mml[r * 2 + 1];
      }
    }
  };
  // Everything that depends on the wave's row blocks: RB of them from rb0 on.
  // Both halves run the same sequence of workgroup barriers.
  auto per_wave = [&](auto rb_count, const int rb0) {
    constexpr int RB = decltype(rb_count)::value;
    constexpr int RBA = RB > 0 ? RB : 1;  // array extents (a wave without rows declares one unused block)
    // Accumulators. o: O^T blocks (unnormalised), touched by the matrix cores
    // only (a VALU rescale of o in the loop would make the register allocator
    // shuttle all of it between accumulation and vector registers every tile).
    // l: the lane's partial row sums of exactly the fp16 probabilities that
    // enter P V. m: the row's reference max (log2 units).
    f32x4 o[8][RBA];
    float m[RBA], l[RBA];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m[rb] = -INFINITY;

    // One tile of this wave's rows in two halves. scores(t): the scores and
    // t = s * kss - m (in place of the scores) with the boundary masks, and the
    // running per-row max of t. back(): turn t into fp16 probabilities, add
    // their row sums and P V into the accumulators.
    f32x4 sacc[2][RBA];
    const char* sl = nullptr;
    float negm[RBA];  // -m, or 0 while m is -inf
    float tmax[RBA];  // the lane's largest t = s * kss - m of its row so far
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) negm[rb] = 0.f;

    auto scores = [&](int t, auto masked) {
      int t0, mode, limit;
      geom(t, t0, mode, limit);
      sl = ring[t % S];

      // S^T = K Q^T: block kb takes tile rows 8(i/4) + 4kb + i%4; k-step outer,
      // so consecutive MFMAs feed independent accumulators
      {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 kf[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int r = 8 * (li >> 2) + 4 * kb + (li & 3);
            kf[kb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(sl + r * RBYTES + 16 * ((4 * ks + lg) ^ lds_swz<false>(r))));
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const bf16x8 qv = __builtin_bit_cast(bf16x8, qsh[((rb0 + rb) * 4 + ks) * 64 + lane]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
              const f32x4 acc = ks == 0 ? zero : sacc[kb][rb];
              sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb], qv, acc, 0, 0, 0);
            }
          }
          // keep one k-step of Q fragments in flight at a time (register budget)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sacc[e >> 2][rb][e & 3] = fmaf(sacc[e >> 2][rb][e & 3], p.scale_log2, negm[rb]);
      }
      if (decltype(masked)::value && mode != 0) {  // boundary tiles: keys past the range, non-ancestors
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint64_t bits = mode == 2 ? tbits_s[(rb0 + rb) * 16 + li] : ~0ull;
          // an edge tile: the row's node i keeps keys >= edge_lo + i
          const int lo = mode == 3 ? tl.edge_lo + (w.row0 + (rb0 + rb) * 16 + li) / p.G : INT_MIN;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = t0 + 8 * lg + e;
            const bool keep = key < limit && key >= lo && ((bits >> ((key - w.P) & 63)) & 1ull);
            sacc[e >> 2][rb][e & 3] = keep ? sacc[e >> 2][rb][e & 3] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          tmax[rb] = fmaxf(fmaxf(tmax[rb], sacc[kb][rb][0]), sacc[kb][rb][1]);
          tmax[rb] = fmaxf(fmaxf(tmax[rb], sacc[kb][rb][2]), sacc[kb][rb][3]);
        }
      }
    };

    auto back = [&]() {
      // P^T fragments (fp16) and their row sums
      f16x8 pw[RBA];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f16x8 pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(sacc[e >> 2][rb][e & 3]));
#pragma unroll
        for (int k = 0; k < 4; ++k)
          l[rb] = __builtin_amdgcn_fdot2(f16x2{pr[2 * k], pr[2 * k + 1]}, f16x2{1, 1}, l[rb], false);
        pw[rb] = pr;
      }
      // O^T += V^T P^T: lane (i, g) reads V rows 8g + e, d = 8i .. 8i+7
      {
        u32x4 vr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * lg + e;
          vr[e] = *reinterpret_cast<const u32x4*>(sl + KBYTES + r * RBYTES + 16 * (li ^ lds_swz<false>(r)));
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          f16x8 vf;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wv = vr[e][db >> 1];
            vf[e] = static_cast<_Float16>(__uint_as_float((db & 1) ? (wv & 0xFFFF0000u) : (wv << 16)));
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pw[rb], o[db][rb], 0, 0, 0);
          }
        }
      }
    };

    // References without rescaling. A row's reference m is set before the loop
    // from the scores of the split's first tile (row max + kMargin). Inside the
    // loop it is only tracked: probabilities stay below 2^6 while no score
    // exceeds m + 6, so p * v_scale stays in fp16 range for any fp16 scale. If
    // a row broke the bound, the split runs again from zero with raised
    // references, so o is never rescaled and the loop carries no branch. Every
    // row's first-tile max is finite: a row sees every key of a prefix tile and,
    // in a block tile, the root.
    constexpr float kMargin = 2.0f;
    auto raise_refs = [&](float margin) -> bool {  // from tmax; true if any row moved
      bool moved = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = fmaxf(tmax[rb], __shfl_xor(tmax[rb], 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__ballot(mx > 6.0f) != 0) {
          moved = true;
          m[rb] = (m[rb] == -INFINITY ? 0.f : m[rb]) + mx + margin;
          negm[rb] = -m[rb];
        }
      }
      return moved;
    };
    if (ntile > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) tmax[rb] = -INFINITY;
      scores(0, std::true_type{});  // with m = -inf (negm = 0): t is the score itself
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = fmaxf(tmax[rb], __shfl_xor(tmax[rb], 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        m[rb] = mx + kMargin;
        negm[rb] = -m[rb];
      }
    }
    float margin = 2.0f * kMargin;
    for (;;) {  // attempts: the first, then one per raise of the references
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        l[rb] = 0.f;
        tmax[rb] = -INFINITY;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // (the work of a step sits in the loop body unconditionally: a
      // conditional accumulation would stop the compiler from updating the
      // matrix-core accumulators in place)
      // full prefix tiles need no masks and come first; a loop of their own
      // keeps the mask code (and its register shuffles) off their path
      auto step = [&](int t, auto masked) {
        wait_tile(t);
        __syncthreads();  // tile t is complete in every pair; slot (t - 1) % S is free
        if (t + S - 1 < ntile) issue(t + S - 1);
        scores(t, masked);
        back();
      };
#pragma nounroll
      for (int t = 0; t < n_full; ++t) step(t, std::false_type{});
#pragma nounroll
      for (int t = n_full; t < ntile; ++t) step(t, std::true_type{});
      for (int t = ntile; t < nt_wg; ++t) __syncthreads();
      // every wave has left the loop (its last wait drained its DMAs) before any
      // ring slot is staged again
      const bool mine = RB > 0 && raise_refs(margin);
      if (!__syncthreads_or(mine)) break;
      margin += kMargin;  // a wider margin on every attempt
#pragma unroll
      for (int u = 0; u < S - 1; ++u)
        if (u < ntile) issue(u);
    }

    // ---- epilogue ----
    // (1) full row sums; (2) the four pairs (four consecutive splits) fold
    // their (m, l, o) into one in LDS, one pair at a time, the two waves of a
    // pair on disjoint rows; (3) a unit covered by this workgroup alone is written
    // out, otherwise one partial per workgroup goes to the workspace and the
    // second launch merges them.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
    }
    __syncthreads();  // every ring is drained
    for (int step = 0; step < NP; ++step) {
      if (pair == step) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int rloc = (rb0 + rb) * 16 + li;
          const float m_old = step ? mml[rloc * 2] : -INFINITY;
          const float l_old = step ? mml[rloc * 2 + 1] : 0.f;
          const float mn = fmaxf(m_old, m[rb]);
          const float a_old = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_old - mn);
          const float a_new = m[rb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[rb] - mn);
#pragma unroll
          for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int idx = (((rb0 + rb) * 8 + db) * 4 + r) * 64 + lane;
              mo[idx] = o[db][rb][r] * a_new + (step ? mo[idx] * a_old : 0.f);
            }
          if (lg == 0) {
            mml[rloc * 2] = mn;
            mml[rloc * 2 + 1] = l[rb] * a_new + l_old * a_old;
          }
        }
      }
      __syncthreads();
    }
  };
  if (h == 0) per_wave(std::integral_constant<int, RB0>{}, 0);
  else per_wave(std::integral_constant<int, RB1>{}, RB0);
  store_out(w, wgi, w.nsplit / NP == 1);  // one partial per workgroup
}

// int8 KV, MFMA path, by phase. A workgroup is NP = 4 wave pairs taking 4
// consecutive key splits of one unit; all RB row blocks of the unit's chunk
// belong to both waves of a pair. The score wave (h = 0) forms S = K Q^T,
// the fp16 probabilities of tile t, their row sums and the v-scaled
// P' = P * v_scale, and hands P' to the value wave (h = 1) through a
// double-buffered LDS block; the value wave accumulates O += P' V for tile
// t - 1 in the same step and issues every staging load of the pair (K tile
// t + 3 with both scale groups, V tile t + 2), so the score wave never waits
// on memory counters. Every K and V byte is converted once, the two waves
// share one SIMD (2 waves per SIMD, 256 registers each), and one workgroup
// barrier per step orders the hand-over.
//
// Codes enter the matrix cores as fp16 of c + 1152 (one v_perm per pair).
// The offset leaves S through the accumulators' start value, -1152 sum_d q_d
// per row, and leaves O through the row sums of P' (a matrix-core product
// with a ones operand): O -= 1152 sum_j P'_j.
constexpr int kMaxAttempts = 8;  // passes over a split, at most (inputs with infinite scores stop there)
// Largest row sum of |q| (times the log2 score scale) that keeps the offset
// code conversion: its extra rounding stays below 4 * 2^-24 * 1279 * 128 *
// k_scale ~ 4e-2 k_scale log2 units (~3e-4 |k|max), under the fp16 rounding of p.
constexpr float kOffsetQ1Max = 128.0f;
//
// The choice between the two conversions is made per workgroup from its rows
// and the kernel is instantiated once per choice (one instantiation holding
// both schedules the offset loop worse): the MODE = kI8Offset launch runs
// every workgroup whose rows keep the offset form and flags the others in
// exact_flags; the MODE = kI8Flagged launch that follows runs the flagged
// ones. A call too small for the offset form's gain to pay for a second
// launch runs every workgroup exact in one MODE = kI8Exact launch.
constexpr int kI8Offset = 0, kI8Flagged = 1, kI8Exact = 2;
template <int RB, int MODE>
__global__ void __launch_bounds__(512) attn_i8_split_kernel(const AttnParams p) {
  constexpr bool EXACT = MODE != kI8Offset;
  constexpr int NP = 4;                      // wave pairs = consecutive key splits of one unit
  constexpr int NW = 2 * NP;                 // waves
  constexpr int D = 128;
  constexpr int RBYTES = D;                  // bytes of one K (or V) row of codes
  constexpr int CH = RBYTES / 16;            // 16-byte chunks per row
  constexpr int KT = 32;                     // keys per tile
  constexpr int KBYTES = KT * RBYTES;        // one K (or V) tile of codes
  constexpr int NK = KBYTES / 1024;          // DMA instructions per K (or V) tile
  constexpr int KSLOT = KBYTES + 128;        // K codes + 32 k-scales + 32 v-scales (fp16)
  constexpr int VSLOT = KBYTES;              // V codes
  // K ring and V ring stages. Loads run three steps ahead: K s + 3 and V s + 2
  // are issued at step s. K s + 3 goes where K s - 1 was (scored a step
  // earlier); V s + 2 goes where V s - 1 was, which the value wave reads into
  // registers just before, so V needs one stage fewer.
  constexpr int SK = 4, SV = 3;
  constexpr int NDK = NK + 1, NDV = NK;      // DMA instructions per staged tile, always all issued
  __shared__ __attribute__((aligned(16))) char kring_all[NP][SK][KSLOT];
  __shared__ __attribute__((aligned(16))) char vring_all[NP][SV][VSLOT];
  __shared__ __attribute__((aligned(16))) u32x4 pbuf_all[NP][2][RB * 64];  // P^T fragments, lane-major
  __shared__ uint64_t tbits_s[RB * 16];
  __shared__ float mref_s[NP][RB * 16];  // the score wave's references and row sums, for the fold
  __shared__ float lref_s[NP][RB * 16];
  __shared__ int s_nt[NP];
  __shared__ int s_bad[NP];  // the value wave's row sums of P' overflowed in this pass
  __shared__ int s_exact;    // this workgroup's rows take the exact code conversion

  const int wgi = xcd_slot(blockIdx.x, p.nwg / NP);
  if (wgi < 0) return;  // whole workgroup
  if constexpr (MODE == kI8Flagged) {
    if (p.exact_flags[wgi] == 0) return;  // the offset launch ran it
  }
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int pair = wave & (NP - 1);  // the pair's two waves sit on one SIMD
  const int h = wave / NP;           // 0: score wave, 1: value wave
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;
  Work w;
  decode(p, wgi * NP + pair, w);  // the pairs share (b, kv head, row chunk)

  for (int r = threadIdx.x; r < RB * 16; r += 64 * NW)
    tbits_s[r] = r < w.nrows ? row_bits(p, w, w.row0 + r) : 1ull;

  const size_t head = (size_t)w.b * p.Hkv + w.kvh;
  const char* kbase = static_cast<const char*>(p.k) + head * p.cap * RBYTES;
  const char* vbase = static_cast<const char*>(p.v) + head * p.cap * RBYTES;
  // value wave, lanes 0-3: k-scales of keys t0 + 8 lane .. +8; lanes 4-7: v-scales
  const uint16_t* sbase = (lane < 4 ? p.ks : p.vs) + head * p.cap;
  const uint32_t kring_lds = lds_u32(kring_all[pair][0]);
  const uint32_t vring_lds = lds_u32(vring_all[pair][0]);
  u32x4(*pbuf)[RB * 64] = pbuf_all[pair];
  // the fold of the four pairs' (m, l, o) reuses the K rings' space
  f32x4* mo = reinterpret_cast<f32x4*>(&kring_all[0][0][0]);  // [RB][8][64] lane-major o blocks
  float* mml = reinterpret_cast<float*>(mo + RB * 8 * 64);      // [RB * 16][2] (m, l)
  static_assert(RB * 32 * 64 * 4 + RB * 16 * 8 <= NP * SK * KSLOT, "fold area");
  const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};

  // Per-lane DMA geometry: piece j of a tile is tile row (64 j + lane) / CH,
  // 16-byte chunk (64 j + lane) % CH of that row (swizzled).
  auto piece_row = [&](int j) { return (64 * j + lane) / CH; };
  auto piece_col = [&](int j) {
    return 16u * static_cast<uint32_t>(((64 * j + lane) % CH) ^ lds_swz<true>(piece_row(j)));
  };
  uint32_t koff[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) koff[j] = static_cast<uint32_t>(piece_row(j) * RBYTES) + piece_col(j);

  // Tile list (full prefix tiles first, then the partial, edge and block ones)
  TileList tl;
  tl.init(p, w, KT);
  const int ntile = tl.ntile;
  const int n_full = tl.n_full;
  auto geom = [&](int t, int& t0, int& mode, int& limit) { tl.geom(t, KT, t0, mode, limit); };
  // Staging loads, issued by the value wave: K tile t (codes + both scale
  // groups: NDK instructions) or V tile t (NDV) into its ring slot. Boundary
  // tiles clamp every row into [t0, limit); a scale group reaching past cap is
  // clamped to start at cap - 8 (cap >= 32).
  auto issue_codes = [&](const char* base, int t, uint32_t dst) {
    int t0, mode, limit;
    geom(t, t0, mode, limit);
    const char* src = base + (size_t)t0 * RBYTES;
    if (mode == 0) {
#pragma unroll
      for (int j = 0; j < NK; ++j) dma16_at(src, koff[j], dst + 1024 * j);
    } else {
      const int lim = limit - 1 - t0;
#pragma unroll
      for (int j = 0; j < NK; ++j)
        dma16_at(src, static_cast<uint32_t>(min(piece_row(j), lim) * RBYTES) + piece_col(j), dst + 1024 * j);
    }
    return t0;
  };
  auto issue_k = [&](int t) {
    const uint32_t dst = kring_lds + static_cast<uint32_t>((t % SK) * KSLOT);
    const int t0 = issue_codes(kbase, t, dst);
    if (lane < 8) dma16v_at(sbase + min(t0 + 8 * (lane & 3), p.cap - 8), dst + KBYTES);
  };
  auto issue_v = [&](int t) { issue_codes(vbase, t, vring_lds + static_cast<uint32_t>((t % SV) * VSLOT)); };
  // Issue order: step s issues K s + 3, then V s + 2 (those that exist); the
  // head stands in for steps -3 .. -1 (K 0; K 1, V 0; K 2, V 1). Before
  // barrier s the value wave needs K s and V s - 1, both issued at step
  // s - 3, so the loads of steps s - 2 and s - 1 may still be in flight:
  // NDK + NDV each while both tiles exist, fewer at the end of the list.
  auto stage_step = [&](int s) __attribute__((always_inline)) {
    if (s + 3 < ntile) issue_k(s + 3);
    if (s + 2 >= 0 && s + 2 < ntile) issue_v(s + 2);
  };
  auto stage_head = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = -3; s < 0; ++s) stage_step(s);
  };
  auto wait_step = [&](int s) {
    const int left = ntile - s;
    if (left >= 3) wait_vmcnt<2 * (NDK + NDV)>();
    else if (left == 2) wait_vmcnt<NDK + 2 * NDV>();
    else if (left == 1) wait_vmcnt<NDV>();
    else wait_vmcnt<0>();
  };
  // the lane group's 8 scales (keys 8g + e of tile t), as fp16 pairs; off 0:
  // k-scales, 64: v-scales
  auto scales = [&](const char* sl, int t0, int off) -> u32x4 {
    if (t0 + KT <= p.cap) return *reinterpret_cast<const u32x4*>(sl + KBYTES + off + 16 * lg);
    const int delta = max(0, t0 + 8 * lg + 8 - p.cap);
    const uint16_t* sp = reinterpret_cast<const uint16_t*>(sl + KBYTES + off + 16 * lg);
    u32x4 r = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e >> 1] |= static_cast<uint32_t>(sp[min(e + delta, 7)]) << (16 * (e & 1));
    return r;
  };

  // The queries enter the matrix cores as fp16, scaled by one power of two
  // per row chunk that brings the chunk's largest |q| into [2^14, 2^15):
  // every bf16 value within 2^28 of that largest converts exactly, and the
  // factor comes back out of the score scale. The chunk's largest row sum of
  // |q| picks the code conversion (see above). The score waves take these
  // statistics while the value waves issue the first loads.
  float qmul = 1.0f, sl2 = p.scale_log2;
  if (h == 0) {
    float amax = 0.f, r1max = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rloc = rb * 16 + li;
      const bool ok = rloc < w.nrows;
      const int row = w.row0 + (ok ? rloc : 0);
      const uint16_t* qrow =
          static_cast<const uint16_t*>(p.q) + ((size_t)(w.o0 + row / p.G) * p.Hq + w.kvh * p.G + row % p.G) * D;
      float r1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * lg + 8 * ks);
        if (!ok) x = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = fabsf(__uint_as_float((e & 1) ? (x[e >> 1] & 0xFFFF0000u) : (x[e >> 1] << 16)));
          amax = fmaxf(amax, a);
          r1 += a;
        }
      }
      r1 += __shfl_xor(r1, 16);
      r1 += __shfl_xor(r1, 32);
      r1max = fmaxf(r1max, r1);
    }
    amax = wave_max(amax);
    r1max = wave_max(r1max);
    int qexp = 0;
    frexpf(amax, &qexp);
    const int qe = __builtin_amdgcn_readfirstlane(amax > 0.f ? min(max(15 - qexp, -126), 126) : 0);
    qmul = ldexpf(1.0f, qe);
    // the score scale with the query factor taken back out (wave-uniform)
    sl2 = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p.scale_log2 * ldexpf(1.0f, -qe))));
    if (pair == 0 && lane == 0) s_exact = (r1max * p.scale_log2 > kOffsetQ1Max || !__builtin_isfinite(r1max)) ? 1 : 0;
  }
  if (h == 1) {
    stage_head();
    wait_step(0);  // K tile 0 has landed: the score wave sets its references from it
  }
  if (lane == 0 && h == 0) s_nt[pair] = ntile;
  __syncthreads();
  if constexpr (!EXACT) {
    const bool skip = s_exact != 0;
    if (threadIdx.x == 0) p.exact_flags[wgi] = skip ? 1 : 0;
    if (skip) {  // left to the exact launch, once this wave's loads have landed
      if (h == 1) wait_vmcnt<0>();
      return;
    }
  }
  int nt_wg = 0;
#pragma unroll
  for (int q = 0; q < NP; ++q) nt_wg = max(nt_wg, s_nt[q]);

  // References without rescaling: set from the scores of the split's first
  // tile (row max + kMargin) and fixed for the pass. If a probability (or its
  // v-scaled copy) overflowed fp16, its row sum is not finite and the split
  // runs again from zero, tracking how far the scores went past the
  // references, and then again with references raised past them. Every row's
  // first-tile max is finite: a row sees every key of a prefix tile and, in a
  // block tile, the root.
  constexpr float kMargin = 2.0f;
  if (h == 0) {
    // ------------------------------------------------------ score wave ----
    // The score wave's chain (S, exp, row sums, P') is the longer one on the
    // shared SIMD: its instructions go first when both waves are ready.
    __builtin_amdgcn_s_setprio(3);
    // Codes enter the matrix cores as fp16 of c + 1152 (one v_perm per pair)
    // with the S accumulators starting at -1152 sum_d q_d, which cancels the
    // offset; the partial sums then run up to ~1279 sum_d |q_d|, so their
    // rounding grows with the rows' |q|. Past kOffsetQ1Max (in log2 score
    // units) the codes are converted exactly instead (one more packed add per
    // pair) and the accumulators start at zero.
    auto score_wave = [&](auto exact_tag) {
    constexpr bool EXACT_CODES = decltype(exact_tag)::value;
    // Q^T fragments in registers: d = 32g + 8ks + e (fp16; a lane's 32 codes
    // of a K row are contiguous)
    f16x8 qf[RB][4];
    f32x4 kinit[RB];  // the S accumulators' start: -1152 sum_d q_d of the lane's row, or 0 (exact codes)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rloc = rb * 16 + li;
      const bool ok = rloc < w.nrows;
      const int row = w.row0 + (ok ? rloc : 0);
      const int node = w.o0 + row / p.G;
      const int qh = w.kvh * p.G + row % p.G;
      const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)node * p.Hq + qh) * D;
      float qsum = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * lg + 8 * ks);
        if (!ok) x = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qf[rb][ks][e] = static_cast<_Float16>(
              __uint_as_float((e & 1) ? (x[e >> 1] & 0xFFFF0000u) : (x[e >> 1] << 16)) * qmul);
          qsum += static_cast<float>(qf[rb][ks][e]);
        }
      }
      qsum += __shfl_xor(qsum, 16);
      qsum += __shfl_xor(qsum, 32);
      const float c = EXACT_CODES ? 0.f : -kCodeBias * qsum;
      kinit[rb] = f32x4{c, c, c, c};
    }
    float negm[RB], tmax[RB], l[RB];  // negm: minus the references (0 for the first tile's raw scores)
    f32x4 sacc[2][RB];
    u32x4 vsc;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) negm[rb] = 0.f;
    // scores of tile t: t = s * kss - m (in place of the scores), boundary
    // masks; with tracking, the running per-row max of t
    auto scores = [&](int t, auto masked, auto track) {
      int t0, mode, limit;
      geom(t, t0, mode, limit);
      const char* sl = kring_all[pair][t % SK];
      const u32x4 ksc = scales(sl, t0, 0);
      vsc = scales(sl, t0, 64);
      if (decltype(masked)::value && mode != 0) {
        // keys at or past the range end (cache rows past the live length
        // among them, whose scales may hold anything) take v-scale 0: their
        // P is 0, and 0 * inf or 0 * NaN would not be
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int key = t0 + 8 * lg + 2 * h;
          vsc[h] &= (key < limit ? 0x0000FFFFu : 0u) | (key + 1 < limit ? 0xFFFF0000u : 0u);
        }
      }
      float kss[8];  // score scale of key 8g + e, log2 units
#pragma unroll
      for (int e = 0; e < 8; ++e) kss[e] = static_cast<float>(__builtin_bit_cast(f16x8, ksc)[e]) * sl2;
      // S^T = K Q^T: block kb takes tile rows 8(i/4) + 4kb + i%4
      u32x4 kraw[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = 8 * (li >> 2) + 4 * kb + (li & 3);
        const char* krow = sl + r * RBYTES;
        const int sw = lds_swz<true>(r);
        kraw[kb][0] = *reinterpret_cast<const u32x4*>(krow + 16 * ((2 * lg) ^ sw)) ^ 0x80808080u;
        kraw[kb][1] = *reinterpret_cast<const u32x4*>(krow + 16 * ((2 * lg + 1) ^ sw)) ^ 0x80808080u;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        f16x8 kf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4& src = kraw[kb][ks >> 1];
          if constexpr (EXACT_CODES) kf[kb] = i8x8_to_f16(src[2 * (ks & 1)], src[2 * (ks & 1) + 1]);
          else kf[kb] = i8x8_to_f16_biased(src[2 * (ks & 1)], src[2 * (ks & 1) + 1]);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb], qf[rb][ks],
                                                                  ks == 0 ? kinit[rb] : sacc[kb][rb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 8; ++e) sacc[e >> 2][rb][e & 3] = fmaf(sacc[e >> 2][rb][e & 3], kss[e], negm[rb]);
      if (decltype(masked)::value && mode != 0) {  // boundary tiles: keys past the range, non-ancestors
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint64_t bits = mode == 2 ? tbits_s[rb * 16 + li] : ~0ull;
          // an edge tile: the row's node i keeps keys >= edge_lo + i
          const int lo = mode == 3 ? tl.edge_lo + (w.row0 + rb * 16 + li) / p.G : INT_MIN;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = t0 + 8 * lg + e;
            const bool keep = key < limit && key >= lo && ((bits >> ((key - w.P) & 63)) & 1ull);
            sacc[e >> 2][rb][e & 3] = keep ? sacc[e >> 2][rb][e & 3] : -INFINITY;
          }
        }
      }
      if constexpr (decltype(track)::value) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            tmax[rb] = fmaxf(fmaxf(tmax[rb], sacc[kb][rb][0]), sacc[kb][rb][1]);
            tmax[rb] = fmaxf(fmaxf(tmax[rb], sacc[kb][rb][2]), sacc[kb][rb][3]);
          }
      }
    };
    // probabilities of the scored tile: p = 2^t in fp16; the row sums of
    // exactly these p (ones x P^T on the matrix cores: every lane gets its
    // row's sum); P' = P * v_scale into P buffer b
    auto hand_over = [&](int b) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f16x8 pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(sacc[e >> 2][rb][e & 3]));
#pragma unroll
        for (int k = 0; k < 4; ++k)
          l[rb] = __builtin_amdgcn_fdot2(f16x2{pr[2 * k], pr[2 * k + 1]}, f16x2{1, 1}, l[rb], false);
        pbuf[b][rb * 64 + lane] = __builtin_bit_cast(u32x4, pr * __builtin_bit_cast(f16x8, vsc));
      }
    };
    // per row block, the furthest any row went past its reference (tracked
    // passes); true if a row went past the bound
    auto past_refs = [&](float (&mx)[RB]) -> bool {
      bool past = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        mx[rb] = fmaxf(tmax[rb], __shfl_xor(tmax[rb], 16));
        mx[rb] = fmaxf(mx[rb], __shfl_xor(mx[rb], 32));
        past |= __ballot(mx[rb] > 6.0f) != 0;
      }
      return past;
    };

    if (ntile > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) tmax[rb] = -INFINITY;
      scores(0, std::true_type{}, std::true_type{});  // with negm = 0: t is the score itself
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = fmaxf(tmax[rb], __shfl_xor(tmax[rb], 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        negm[rb] = -(mx + kMargin);
      }
    }
    float margin = 2.0f * kMargin;
    for (int attempt = 0;; ++attempt) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        tmax[rb] = -INFINITY;
        l[rb] = 0.f;
      }
      // (the work of a step sits in the loop body unconditionally: a
      // conditional accumulation would stop the compiler from updating the
      // matrix-core accumulators in place)
      auto step = [&](int t, auto masked, auto track) {
        __syncthreads();  // K tile t landed; P buffer t % 2 was read a step ago
        scores(t, masked, track);
        hand_over(t & 1);
      };
      if (attempt == 0) {
        // full prefix tiles need no masks and come first; a loop of their
        // own keeps the mask code (and its register shuffles) off their path
#pragma nounroll
        for (int t = 0; t < n_full; ++t) step(t, std::false_type{}, std::false_type{});
#pragma nounroll
        for (int t = n_full; t < ntile; ++t) step(t, std::true_type{}, std::false_type{});
      } else {
#pragma nounroll
        for (int t = 0; t < ntile; ++t) step(t, std::true_type{}, std::true_type{});
      }
      for (int t = ntile; t <= nt_wg; ++t) __syncthreads();  // the value wave's last step, padding
      bool bad = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bad |= !__builtin_isfinite(l[rb]);
      float mx[RB];
      const bool past = attempt > 0 && past_refs(mx);
      const bool redo = __syncthreads_or(bad || past) && attempt + 1 < kMaxAttempts;
      if (!redo) break;
      if (attempt > 0) {
        // raise the rows that went past the bound to put each row's largest
        // score at the usual kMargin below its reference (the scores are
        // recomputed identically, so neither P nor P' can overflow again,
        // and P' of small-v-scale keys keeps the first pass's distance from
        // fp16's subnormal range); an overflow with none of them came from
        // P * v_scale: lower every row of this split by the growing margin
        const bool lower_all = !past && (__ballot(bad) != 0 || s_bad[pair] != 0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if (__ballot(mx[rb] > 6.0f) != 0) negm[rb] -= mx[rb] + kMargin;
          else if (lower_all) negm[rb] -= margin;
        }
      }
      margin += kMargin;  // a wider margin on every pass
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
      if (lg == 0) {
        mref_s[pair][rb * 16 + li] = ntile > 0 ? -negm[rb] : -INFINITY;  // -inf: an empty split
        lref_s[pair][rb * 16 + li] = l[rb];
      }
    }
    __syncthreads();  // references visible, rings idle
    for (int step = 0; step < NP; ++step) __syncthreads();  // the value waves fold
    };
    score_wave(std::integral_constant<bool, EXACT>{});
  } else {
    // ------------------------------------------------------ value wave ----
    f32x4 o[8][RB], osum[RB];
    // V tile t into registers, transposed by the read (ds_read_b64_tr_b8): the
    // 16 lanes of lane group g address both 8-byte halves of chunk db of rows
    // 8 g .. 8 g + 7 (lane r: row 8 g + r / 2, half r % 2) and lane i receives
    // byte i % 8 of half i / 8 of each of those rows, so a[db] holds the codes
    // of keys 8 g + e (byte e) at d = 16 db + i: one d-block of V^T. The slot
    // is free for the next DMA once these reads returned.
    uint32_t a[8][2];
    auto load_v = [&](int t) {
      const int r = 8 * lg + (li >> 1);
      const char* rowp = vring_all[pair][t % SV] + r * RBYTES + 8 * (li & 1);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(rowp + 16 * (db ^ lds_swz<true>(r))));
        a[db][0] = static_cast<uint32_t>(x[0]) ^ 0x80808080u;
        a[db][1] = static_cast<uint32_t>(x[1]) ^ 0x80808080u;
      }
      wait_lgkmcnt0();
    };
    // O^T += V^T P'^T for the loaded tile from P buffer b: d-block db's V^T
    // fragment is a[db] as fp16 of c + 1152, four d-blocks at a time
    // (register budget: o holds 32 RB)
    auto accumulate = [&](int b) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f16x8 vf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vf[j] = i8x8_to_f16_biased(a[4 * hh + j][0], a[4 * hh + j][1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f16x8 pw = __builtin_bit_cast(f16x8, pbuf[b][rb * 64 + lane]);
          if (hh == 0) osum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pw, osum[rb], 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[4 * hh + j][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[j], pw, o[4 * hh + j][rb], 0, 0, 0);
        }
      }
    };
    for (int attempt = 0;; ++attempt) {  // passes, in step with the score wave
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        osum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (attempt > 0) stage_head();
      wait_step(0);
      __syncthreads();  // step 0: K tile 0 has landed
      stage_step(0);
#pragma nounroll
      for (int s = 1; s <= ntile; ++s) {
        wait_step(s);  // K tile s and V tile s - 1 have landed
        __syncthreads();  // P of tile s - 1 is in buffer (s - 1) % 2
        load_v(s - 1);
        stage_step(s);  // V s + 2 reuses the slot of V s - 1
        accumulate((s - 1) & 1);
      }
      for (int s = ntile + 1; s <= nt_wg; ++s) __syncthreads();
      bool bad = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bad |= !__builtin_isfinite(osum[rb][0]);
      const bool bad_w = __ballot(bad) != 0;
      if (lane == 0) s_bad[pair] = bad_w ? 1 : 0;
      const bool redo = __syncthreads_or(bad) && attempt + 1 < kMaxAttempts;
      if (!redo) break;
    }
    // take the code offset back out of O
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[db][rb][j] = fmaf(-kCodeBias, osum[rb][j], o[db][rb][j]);
    __syncthreads();  // references and row sums visible, rings idle
    // the four pairs (four consecutive splits) fold their (m, l, o) into one,
    // one pair at a time
    for (int step = 0; step < NP; ++step) {
      if (pair == step) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int rloc = rb * 16 + li;
          const float m_new = mref_s[pair][rloc];
          const float l_new = lref_s[pair][rloc];
          const float m_old = step ? mml[rloc * 2] : -INFINITY;
          const float l_old = step ? mml[rloc * 2 + 1] : 0.f;
          const float mn = fmaxf(m_old, m_new);
          const float a_old = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_old - mn);
          const float a_new = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_new - mn);
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const int idx = (rb * 8 + db) * 64 + lane;
            mo[idx] = step ? o[db][rb] * a_new + mo[idx] * a_old : o[db][rb] * a_new;
          }
          if (lg == 0) {
            mml[rloc * 2] = mn;
            mml[rloc * 2 + 1] = l_new * a_new + l_old * a_old;
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- epilogue ----
  // A unit covered by this workgroup alone is written out, otherwise one
  // partial per workgroup goes to the workspace and a second launch merges
  // them.
  const int nwg_unit = w.nsplit / NP;
  // Row-major stores, four consecutive d per thread (coalesced); o sits in LDS
  // in the MFMA lane order: row 16 rb + i, d = 16 db + 4 g + r is element r of
  // block (rb * 8 + db) * 64 + 16 g + i, so four consecutive d are one block
  // entry.
  for (int flat = 4 * threadIdx.x; flat < w.nrows * D; flat += 4 * 64 * NW) {
    const int rloc = flat / D, d0 = flat % D;
    const int rb = rloc >> 4, i = rloc & 15;
    f32x4 v = mo[(rb * 8 + (d0 >> 4)) * 64 + 16 * ((d0 >> 2) & 3) + i];
    if (nwg_unit == 1) {
      const int row = w.row0 + rloc;
      const int node = w.o0 + row / p.G;
      const int qh = w.kvh * p.G + row % p.G;
      *reinterpret_cast<f32x4*>(p.out + ((size_t)node * p.Hq + qh) * D + d0) = v / mml[rloc * 2 + 1];
    } else {
      *reinterpret_cast<f32x4*>(p.part_o + ((size_t)wgi * p.rows_chunk + rloc) * D + d0) = v;
    }
  }
  if (nwg_unit > 1) {
    for (int r = threadIdx.x; r < w.nrows; r += 64 * NW) {
      p.part_ml[((size_t)wgi * p.rows_chunk + r) * 2] = mml[r * 2];
      p.part_ml[((size_t)wgi * p.rows_chunk + r) * 2 + 1] = mml[r * 2 + 1];
    }
  }
}

// bf16 KV with more than 16 * kMfmaMaxRB rows per KV head, MFMA path, by
// phase. A workgroup is NP = 4 wave pairs taking up to 4 row chunks (of at
// most RBMAX row blocks each) of one (sequence, KV head, key split) side by
// side, so each K/V byte is read once for up to 4 * 80 rows; the pairs share
// one ring of 32-key K and V tiles. The score wave of a pair holds its chunk's
// Q^T in registers, forms S = K Q^T, the fp16 probabilities and their row sums
// and hands P to its value wave through a double-buffered LDS block. The value
// wave accumulates O += P V for the previous tile and issues its quarter of
// every staging load; V is converted to fp16 once per workgroup, each value
// wave building two of the eight d-blocks of the tile's V^T fragments. One
// workgroup barrier per step orders the hand-overs. Both waves of a pair run
// the variant compiled for the pair's own row-block count.
template <int RBMAX>
__global__ void __launch_bounds__(512) attn_bf16_split_kernel(const AttnParams p) {
  constexpr int NP = 4;                 // wave pairs = row chunks side by side
  constexpr int NW = 2 * NP;
  constexpr int D = 128;
  constexpr int RBYTES = 2 * D;         // one bf16 K (or V) row
  constexpr int CH = RBYTES / 16;       // 16-byte chunks per row
  constexpr int KT = 32;                // keys per tile
  constexpr int KBYTES = KT * RBYTES;   // one K (or V) tile
  constexpr int NK = KBYTES / 1024;     // DMA instructions per K (or V) tile
  constexpr int NKW = NK / NP;          // ... per value wave
  constexpr int AHEAD = 3;              // tiles staged ahead of the one in use
  constexpr int S = AHEAD + 1;          // ring stages (K and V alike)
  constexpr int NDS = 2 * NKW;          // DMA instructions of one value wave per step
  __shared__ __attribute__((aligned(16))) char kring[S][KBYTES];
  __shared__ __attribute__((aligned(16))) char vring[S][KBYTES];
  __shared__ __attribute__((aligned(16))) u32x4 vT[2][8 * 64];  // fp16 V^T fragments, by d-block
  __shared__ __attribute__((aligned(16))) u32x4 pbuf_all[NP][2][RBMAX * 64];
  __shared__ uint64_t tbits_all[NP][RBMAX * 16];
  __shared__ float mref_all[NP][RBMAX * 16];
  __shared__ float lref_all[NP][RBMAX * 16];

  // Workgroups are dealt to the XCDs round-robin in launch order: sequences
  // of very different lengths then spread their work over every XCD (no two
  // workgroups share K/V, so nothing is lost by leaving the XCD-contiguous
  // map); the launch order runs the short last splits at the end
  if (static_cast<int>(blockIdx.x) >= p.nwg / NP) return;  // whole workgroup
  const int wgi = wide_order(p, static_cast<int>(blockIdx.x));
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int pair = wave & (NP - 1);  // the pair's two waves sit on one SIMD
  const int h = wave / NP;           // 0: score wave, 1: value wave
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lg = lane >> 4;
  Work w;
  decode(p, wgi * NP + pair, w);  // the pairs share (b, kv head, split); row chunk rc = pair's slot
  const int nrb = (w.nrows + 15) / 16;  // <= RBMAX; 0 for a padding chunk
  uint64_t* tbits_s = tbits_all[pair];
  u32x4(*pbuf)[RBMAX * 64] = pbuf_all[pair];

  for (int r = lane + (h ? 64 : 0); r < RBMAX * 16; r += 128)
    tbits_s[r] = r < w.nrows ? row_bits(p, w, w.row0 + r) : 1ull;

  const size_t head = (size_t)w.b * p.Hkv + w.kvh;
  const char* kbase = static_cast<const char*>(p.k) + head * p.cap * RBYTES;
  const char* vbase = static_cast<const char*>(p.v) + head * p.cap * RBYTES;
  const uint32_t kring_lds = lds_u32(kring[0]);
  const uint32_t vring_lds = lds_u32(vring[0]);

  // Per-lane DMA geometry: piece j of a tile is tile row (64 j + lane) / CH,
  // 16-byte chunk (64 j + lane) % CH of that row (swizzled); value wave q
  // stages pieces NKW * q .. NKW * q + NKW - 1 of every K and V tile.
  const int j0 = NKW * pair;
  auto piece_row = [&](int j) { return (64 * j + lane) / CH; };
  auto piece_col = [&](int j) {
    return 16u * static_cast<uint32_t>(((64 * j + lane) % CH) ^ lds_swz<false>(piece_row(j)));
  };
  uint32_t koff[NKW];
#pragma unroll
  for (int j = 0; j < NKW; ++j) koff[j] = static_cast<uint32_t>(piece_row(j0 + j) * RBYTES) + piece_col(j0 + j);

  // Tile list (full prefix tiles first, then the partial, edge and block
  // ones); every pair has the same
  TileList tl;
  tl.init(p, w, KT);
  const int ntile = tl.ntile;
  const int n_full = tl.n_full;
  auto geom = [&](int t, int& t0, int& mode, int& limit) { tl.geom(t, KT, t0, mode, limit); };
  // this value wave's pieces of tile t of K (or V) into ring slot t % S;
  // boundary tiles clamp every row into [t0, limit)
  auto issue_tile = [&](const char* base, uint32_t ring_lds, int t) {
    int t0, mode, limit;
    geom(t, t0, mode, limit);
    const char* src = base + (size_t)t0 * RBYTES;
    const uint32_t dst = ring_lds + static_cast<uint32_t>((t % S) * KBYTES + 1024 * j0);
    if (mode == 0) {
#pragma unroll
      for (int j = 0; j < NKW; ++j) dma16_at(src, koff[j], dst + 1024 * j);
    } else {
      const int lim = limit - 1 - t0;
#pragma unroll
      for (int j = 0; j < NKW; ++j)
        dma16_at(src, static_cast<uint32_t>(min(piece_row(j0 + j), lim) * RBYTES) + piece_col(j0 + j),
                 dst + 1024 * j);
    }
  };
  // step s stages K and V of tile s + AHEAD; the head stands in for steps
  // -AHEAD .. -1. Before barrier s the value waves need K s and V s (staged at
  // step s - AHEAD): the loads of the AHEAD - 1 later steps may be in flight.
  auto stage = [&](int s) __attribute__((always_inline)) {
    if (s + AHEAD < ntile) {
      issue_tile(kbase, kring_lds, s + AHEAD);
      issue_tile(vbase, vring_lds, s + AHEAD);
    }
  };
  auto stage_head = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < AHEAD; ++t)
      if (t < ntile) {
        issue_tile(kbase, kring_lds, t);
        issue_tile(vbase, vring_lds, t);
      }
  };
  static_assert(AHEAD >= 1 && AHEAD <= 5, "wait_step covers up to four later steps");
  auto wait_step = [&](int s) {
    const int later = min(AHEAD - 1, ntile - 1 - s);  // steps after s whose tiles are staged
    if (later >= 4) wait_vmcnt<4 * NDS>();
    else if (later == 3) wait_vmcnt<3 * NDS>();
    else if (later == 2) wait_vmcnt<2 * NDS>();
    else if (later == 1) wait_vmcnt<NDS>();
    else wait_vmcnt<0>();
  };

  if (h == 1) {
    stage_head();
    if (ntile > 0) wait_step(0);
  }
  __syncthreads();

  constexpr float kMargin = 2.0f;
  auto score_wave = [&](auto rb_count) {
    constexpr int RB = decltype(rb_count)::value;
    constexpr int RBA = RB > 0 ? RB : 1;
    // Q^T fragments in registers: d = 32 ks + 8 g + e (bf16)
    bf16x8 qf[RBA][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rloc = rb * 16 + li;
      const bool ok = rloc < w.nrows;
      const int row = w.row0 + (ok ? rloc : 0);
      const uint16_t* qrow =
          static_cast<const uint16_t*>(p.q) + ((size_t)(w.o0 + row / p.G) * p.Hq + w.kvh * p.G + row % p.G) * D;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg);
        if (!ok) x = u32x4{0, 0, 0, 0};
        qf[rb][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
    float negm[RBA], tmax[RBA], l[RBA];
    f32x4 sacc[2][RBA];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) negm[rb] = 0.f;
    // scores of tile t: t = s * scale - m in place of the scores, boundary
    // masks; with tracking, the running per-row max of t
    auto scores = [&](int t, auto masked, auto track) {
      int t0, mode, limit;
      geom(t, t0, mode, limit);
      const char* sl = kring[t % S];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 kf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = 8 * (li >> 2) + 4 * kb + (li & 3);
          kf[kb] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(sl + r * RBYTES + 16 * ((4 * ks + lg) ^ lds_swz<false>(r))));
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb], qf[rb][ks], ks == 0 ? zero : sacc[kb][rb],
                                                                   0, 0, 0);
          }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 8; ++e) sacc[e >> 2][rb][e & 3] = fmaf(sacc[e >> 2][rb][e & 3], p.scale_log2, negm[rb]);
      if (decltype(masked)::value && mode != 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint64_t bits = mode == 2 ? tbits_s[rb * 16 + li] : ~0ull;
          // an edge tile: the row's node i keeps keys >= edge_lo + i
          const int lo = mode == 3 ? tl.edge_lo + (w.row0 + rb * 16 + li) / p.G : INT_MIN;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = t0 + 8 * lg + e;
            const bool keep = key < limit && key >= lo && ((bits >> ((key - w.P) & 63)) & 1ull);
            sacc[e >> 2][rb][e & 3] = keep ? sacc[e >> 2][rb][e & 3] : -INFINITY;
          }
        }
      }
      if constexpr (decltype(track)::value) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            tmax[rb] = fmaxf(fmaxf(tmax[rb], sacc[kb][rb][0]), sacc[kb][rb][1]);
            tmax[rb] = fmaxf(fmaxf(tmax[rb], sacc[kb][rb][2]), sacc[kb][rb][3]);
          }
      }
    };
    // fp16 probabilities of the scored tile into P buffer b, and their row sums
    auto hand_over = [&](int b) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f16x8 pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(sacc[e >> 2][rb][e & 3]));
#pragma unroll
        for (int k = 0; k < 4; ++k)
          l[rb] = __builtin_amdgcn_fdot2(f16x2{pr[2 * k], pr[2 * k + 1]}, f16x2{1, 1}, l[rb], false);
        pbuf[b][rb * 64 + lane] = __builtin_bit_cast(u32x4, pr);
      }
    };
    auto past_refs = [&](float (&mx)[RBA]) -> bool {
      bool past = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        mx[rb] = fmaxf(tmax[rb], __shfl_xor(tmax[rb], 16));
        mx[rb] = fmaxf(mx[rb], __shfl_xor(mx[rb], 32));
        past |= __ballot(mx[rb] > 6.0f) != 0;
      }
      return past;
    };
    if (ntile > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) tmax[rb] = -INFINITY;
      scores(0, std::true_type{}, std::true_type{});  // with negm = 0: t is the score itself
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = fmaxf(tmax[rb], __shfl_xor(tmax[rb], 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        negm[rb] = -(mx + kMargin);
      }
    }
    float margin = 2.0f * kMargin;
    for (int attempt = 0;; ++attempt) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        tmax[rb] = -INFINITY;
        l[rb] = 0.f;
      }
      auto step = [&](int t, auto masked, auto track) {
        __syncthreads();  // K tile t landed; P buffer t % 2 was read a step ago
        scores(t, masked, track);
        hand_over(t & 1);
      };
      if (attempt == 0) {
#pragma nounroll
        for (int t = 0; t < n_full; ++t) step(t, std::false_type{}, std::false_type{});
#pragma nounroll
        for (int t = n_full; t < ntile; ++t) step(t, std::true_type{}, std::false_type{});
      } else {
#pragma nounroll
        for (int t = 0; t < ntile; ++t) step(t, std::true_type{}, std::true_type{});
      }
      __syncthreads();  // the value waves' last step
      bool bad = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bad |= !__builtin_isfinite(l[rb]);
      float mx[RBA];
      const bool past = attempt > 0 && RB > 0 && past_refs(mx);
      const bool redo = __syncthreads_or(bad || past) && attempt + 1 < kMaxAttempts;
      if (!redo) break;
      if (attempt > 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (__ballot(mx[rb] > 6.0f) != 0) negm[rb] -= mx[rb] + margin;
      }
      margin += kMargin;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
      if (lg == 0) {
        mref_all[pair][rb * 16 + li] = ntile > 0 ? -negm[rb] : -INFINITY;  // -inf: an empty split
        lref_all[pair][rb * 16 + li] = l[rb];
      }
    }
    __syncthreads();  // references and row sums visible
  };

  auto value_wave = [&](auto rb_count) {
    constexpr int RB = decltype(rb_count)::value;
    // its instructions go first when both waves of the pair are ready: the
    // score wave's exponentials then run beside these products (-2% against
    // no priority, -1% against the score wave first)
    __builtin_amdgcn_s_setprio(3);
    constexpr int RBA = RB > 0 ? RB : 1;
    f32x4 o[8][RBA];
    // V^T fragments of V tile t as fp16 into vT[t & 1]: fragment (db, lane
    // (i, g)) holds V[8g + e][8i + db], e = 0..7. Value wave q builds the
    // fragments of lanes g = q, i.e. keys 8 q .. 8 q + 7: its lane (i, j)
    // reads dword j of 16-byte chunk i of each of those 8 rows (a whole row
    // per read, free of bank conflicts) and writes d-blocks 2 j and 2 j + 1.
    auto convert_v = [&](int t) {
      const char* vt0 = vring[t % S];
      f16x8 f0, f1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * pair + e;
        const uint32_t x = *reinterpret_cast<const uint32_t*>(vt0 + r * RBYTES + 16 * (li ^ lds_swz<false>(r)) + 4 * lg);
        f0[e] = static_cast<_Float16>(__uint_as_float(x << 16));
        f1[e] = static_cast<_Float16>(__uint_as_float(x & 0xFFFF0000u));
      }
      vT[t & 1][(2 * lg) * 64 + 16 * pair + li] = __builtin_bit_cast(u32x4, f0);
      vT[t & 1][(2 * lg + 1) * 64 + 16 * pair + li] = __builtin_bit_cast(u32x4, f1);
    };
    // O^T += V^T P^T for tile t from vT[t & 1] and P buffer t & 1
    auto accumulate = [&](int t) {
      f16x8 pw[RBA];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) pw[rb] = __builtin_bit_cast(f16x8, pbuf[t & 1][rb * 64 + lane]);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f16x8 vf = __builtin_bit_cast(f16x8, vT[t & 1][db * 64 + lane]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pw[rb], o[db][rb], 0, 0, 0);
      }
    };
    for (int attempt = 0;; ++attempt) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (attempt > 0) {
        stage_head();
        if (ntile > 0) wait_step(0);
      }
#pragma nounroll
      for (int s = 0; s <= ntile; ++s) {
        if (s > 0 && s < ntile) wait_step(s);  // K and V of tile s have landed (step 0 waited above)
        __syncthreads();  // and every pair's P of tile s - 1 is in its buffer
        stage(s);
        if (s > 0) accumulate(s - 1);  // V^T of tile s - 1 and its P: MFMAs issued first
        if (s < ntile) convert_v(s);    // into the other V^T buffer while they run
      }
      const bool redo = __syncthreads_or(false) && attempt + 1 < kMaxAttempts;
      if (!redo) break;
    }
    __syncthreads();  // the score wave's references and row sums
    if (RB == 0) return;
    // output rows: lane (i, g) holds d = 32 g + 8 r + db of row 16 rb + i in
    // o[db][rb][r]; the unit's output when one split covers it, else a
    // partial of this chunk
    const bool whole = w.nsplit == 1;
    const int slot = wgi * NP + pair;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rloc = rb * 16 + li;
      if (rloc >= w.nrows) continue;
      const float m = mref_all[pair][rloc];
      const float lsum = lref_all[pair][rloc];
      float* dst;
      float scl;
      if (whole) {
        const int row = w.row0 + rloc;
        dst = p.out + ((size_t)(w.o0 + row / p.G) * p.Hq + w.kvh * p.G + row % p.G) * D;
        scl = 1.0f / lsum;
      } else {
        const size_t pr = (size_t)slot * p.rows_chunk + rloc;
        dst = p.part_o + pr * D;
        scl = 1.0f;
        if (lg == 0) {
          p.part_ml[pr * 2] = m;
          p.part_ml[pr * 2 + 1] = lsum;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v0, v1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v0[u] = o[u][rb][r] * scl;
          v1[u] = o[4 + u][rb][r] * scl;
        }
        *reinterpret_cast<f32x4*>(dst + 32 * lg + 8 * r) = v0;
        *reinterpret_cast<f32x4*>(dst + 32 * lg + 8 * r + 4) = v1;
      }
    }
  };

  switch (nrb) {
#define TTV_BF16_ROLE(N)                                                            \
  case N:                                                                           \
    if constexpr (N <= RBMAX) {                                                     \
      if (h == 0) score_wave(std::integral_constant<int, N>{});                     \
      else value_wave(std::integral_constant<int, N>{});                            \
    }                                                                               \
    break;
    TTV_BF16_ROLE(0)
    TTV_BF16_ROLE(1)
    TTV_BF16_ROLE(2)
    TTV_BF16_ROLE(3)
    TTV_BF16_ROLE(4)
    default:
      if (h == 0) score_wave(std::integral_constant<int, RBMAX>{});
      else value_wave(std::integral_constant<int, RBMAX>{});
      break;
#undef TTV_BF16_ROLE
  }
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
  // window band: row r (node t, cache row P + t) keeps keys >= P + t - window + 1
  int lo[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    lo[r] = (p.window > 0 && r < w.nrows) ? w.P + (w.row0 + r) / p.G - p.window + 1 : INT_MIN;

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
      if (!valid || key < lo[r] || (mode == 2 && !((bits[r] >> (key - w.P)) & 1ull))) x = -INFINITY;
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
}

// ------------------------------------------------------------- planning ----

struct AttnPlan {
  bool mfma;
  bool wide;  // bf16 MFMA with the four pairs of a workgroup on four row chunks of one split
  int rb;
  AttnParams prm;  // everything except pointers
  int nunits;
  bool merge;  // some unit has more than one partial
  bool i8_one_launch;  // int8: every workgroup takes the exact conversion in a single launch
  size_t off_ml, off_o, off_flags, ws_bytes;
};

static ttv_status plan_attention(const ttv_batch* batch, int Hq, const ttv_kv_layer* L, int q_dtype,
                                 AttnPlan& pl, int window = 0) {
  ttv_status s = check_batch(batch, false);
  if (s != TTV_OK) return s;
  TTV_REQUIRE(window >= 0, TTV_ERR_INVALID, "tree_verify_attention: window %d < 1", window);
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
  // a window on the matrix cores: at least 64 keys (so no block key of a
  // tree of at most 64 nodes leaves the band), and every sequence whose
  // first keys are hidden from some rows (at most two 32-key edge tiles)
  // also has a whole tile past them, which the MFMA kernels score first
  bool window_mfma = window == 0 || window >= 64;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    const int P = batch->hist_len_h[b];
    TTV_REQUIRE((int64_t)P + T <= L->cap, TTV_ERR_INVALID,
                "tree_verify_attention: sequence %d needs P + T = %d rows, cache holds %d", b, P + T, L->cap);
    max_rows = T * G > max_rows ? T * G : max_rows;
    const int ks = hist_key_start(P, window);
    const int ph = P - ks;  // history keys the sequence's rows read
    maxP = ph > maxP ? ph : maxP;
    if (window > 0) {
      const int edge_end = std::min(P - window + T, P);  // node i keeps keys >= P - window + 1 + i
      const int n_edge = edge_end > ks ? (edge_end - ks + 31) / 32 : 0;
      if (n_edge > 0 && ph < 32 * (n_edge + 1)) window_mfma = false;
    }
  }
  // fewer than 16 rows still take the matrix cores, with the block's missing
  // rows as zero queries: the VALU kernel's one wave per 16 rows and split
  // would leave most of the chip idle
  pl.mfma = bf && L->D == 128 && max_rows >= 1 && L->cap >= 32 && window_mfma;
  pl.wide = pl.mfma && L->dtype != TTV_I8 && max_rows > 16 * kMfmaMaxRB;
  if (pl.wide) {
    // up to four balanced chunks of at most 80 rows side by side (more rows
    // take further groups of four)
    const int ngrp = (max_rows + 4 * 16 * kWideMaxRB - 1) / (4 * 16 * kWideMaxRB);
    const int per = (max_rows + 4 * ngrp - 1) / (4 * ngrp);
    pl.rb = (per + 15) / 16;
    if (pl.rb < 2) pl.rb = 2;
  } else if (pl.mfma) {
    // balanced row chunks of at most 96 rows (int8: 80): pl.rb row blocks
    const int max_rows_chunk = 16 * (L->dtype == TTV_I8 ? kI8MaxRB : kMfmaMaxRB);
    const int nch = (max_rows + max_rows_chunk - 1) / max_rows_chunk;
    const int per = (max_rows + nch - 1) / nch;
    pl.rb = (per + 15) / 16;
    if (L->dtype != TTV_I8 && pl.rb < 2) pl.rb = 2;  // one block per wave of a pair at least
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
  // rows per chunk of each sequence: the launch's chunk, or for the wide
  // layout the sequence's own row blocks spread over groups of four chunks
  // (so a small tree keeps its rows on few waves and a large one on all)
  auto chunk_rows = [&](int rows) -> int {
    if (!pl.wide || rows == 0) return p.rows_chunk;
    const int nrb = (rows + 15) / 16;
    const int ngrp = (nrb + 4 * kWideMaxRB - 1) / (4 * kWideMaxRB);
    return 16 * ((nrb + 4 * ngrp - 1) / (4 * ngrp));
  };
  int max_rch = 0;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    p.rchunk[b] = chunk_rows(T * G);
    max_rch = p.rchunk[b] > max_rch ? p.rchunk[b] : max_rch;
  }
  if (pl.wide) p.rows_chunk = max_rch;  // the partials' row stride
  // wide: every (kv head, split) takes its chunk count rounded up to 4 slots
  // (one workgroup per 4)
  p.wide = pl.wide ? 1 : 0;
  p.window = window;
  int64_t work = 0;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    const int rc = (T * G + p.rchunk[b] - 1) / p.rchunk[b];
    const int P = batch->hist_len_h[b];
    const int ph = P - hist_key_start(P, window);
    work += (int64_t)p.Hkv * (pl.wide ? (rc + 3) / 4 : rc) * (ph > 0 ? ph : 1);
  }
  // a wide workgroup's partial is up to 320 rows of fp32: its split is kept
  // long (about two workgroups per compute unit; with the short last splits
  // dispatched at the end the tail stays small)
  int64_t sl = (work + (pl.wide ? kWideTargetWG : kTargetWG) - 1) / (pl.wide ? kWideTargetWG : kTargetWG);
  const int64_t min_sl = (maxP + kMaxSplits - 1) / kMaxSplits;
  if (sl < min_sl) sl = min_sl;
  // at least four 32-key tiles: short histories still spread over several
  // workgroups, and a window's first split holds its (at most two) edge
  // tiles and a whole tile past them
  if (sl < 128) sl = 128;
  sl = (sl + 63) / 64 * 64;
  p.split_len = static_cast<int>(sl);
  // MFMA workgroups are 4 wave pairs = 4 consecutive key splits of one unit,
  // so a unit's split count is padded to a multiple of 4 (padding splits are
  // empty); wide workgroups take 4 row chunks of one split instead
  p.split_pad = pl.mfma && !pl.wide ? 4 : 1;
  int wg = 0, units = 0;
  pl.merge = false;
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    const int P = batch->hist_len_h[b];
    const int rc = (T * G + p.rchunk[b] - 1) / p.rchunk[b];
    const int ph = P - hist_key_start(P, window);
    const int ns0 = ph > 0 ? (ph + p.split_len - 1) / p.split_len : 1;
    const int ns = (ns0 + p.split_pad - 1) / p.split_pad * p.split_pad;
    // the merge launch keeps one weight per (row, partial) of its rows in LDS
    TTV_REQUIRE(ns / p.split_pad <= kMaxSplits, TTV_ERR_INVALID,
                "tree_verify_attention: sequence %d would need %d partials per unit (at most %d)", b,
                ns / p.split_pad, kMaxSplits);
    p.node_off[b] = batch->node_off_h[b];
    p.hist_len[b] = P;
    p.wg_off[b] = wg;
    p.unit_off[b] = units;
    wg += p.Hkv * ns * (pl.wide ? (rc + 3) / 4 * 4 : rc);
    units += p.Hkv * rc;
    if (rc > 0 && ns / p.split_pad > 1) pl.merge = true;
  }
  p.node_off[B] = batch->node_off_h[B];
  p.wg_off[B] = wg;
  p.unit_off[B] = units;
  // int8: below ~512 MB of K/V a call's kernel runs a few hundred µs or less,
  // where the offset form's few percent are worth less than the exact
  // launch that follows it (~5 µs): run everything exact in one launch
  {
    int64_t kv_rows = 0;
    for (int b = 0; b < B; ++b) {
      const int P = batch->hist_len_h[b];
      kv_rows += (int64_t)p.Hkv * (P - hist_key_start(P, window) + batch->node_off_h[b + 1] - batch->node_off_h[b]);
    }
    pl.i8_one_launch = L->dtype == TTV_I8 && kv_rows * (2 * L->D + 4) < (int64_t{512} << 20);
  }
  if (pl.wide) {
    // dispatch order (wide_order): full-length splits first, then the last
    // splits by descending cost (keys times a row-block weight)
    int32_t order[TTV_MAX_BATCH];
    int64_t cost[TTV_MAX_BATCH];
    int nfull = 0;
    for (int b = 0; b < B; ++b) {
      const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
      const int rc = (T * G + p.rchunk[b] - 1) / p.rchunk[b];
      const int ns = seq_splits(p, b);
      const int ks = hist_key_start(p.hist_len[b], window);
      const int last_keys = p.hist_len[b] - ks - (ns - 1) * p.split_len + T;
      p.full_off[b] = nfull;
      nfull += p.Hkv * (ns - 1) * ((rc + 3) / 4);
      cost[b] = (int64_t)last_keys * (6 + p.rchunk[b] / 16);
      order[b] = b;
    }
    p.full_off[B] = nfull;
    std::stable_sort(order, order + B, [&](int x, int y) { return cost[x] > cost[y]; });
    int nlast = 0;
    for (int k = 0; k < B; ++k) {
      const int b = order[k];
      const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
      const int rc = (T * G + p.rchunk[b] - 1) / p.rchunk[b];
      p.last_key[k] = (nlast << 8) | b;
      nlast += p.Hkv * ((rc + 3) / 4);
    }
    p.last_key[B] = nlast << 8;
    TTV_REQUIRE(nfull + nlast == wg / 4 && nlast < (1 << 22), TTV_ERR_INVALID,
                "tree_verify_attention: %d workgroups exceed the dispatch-order table", wg / 4);
  }
  p.nwg = wg;
  pl.nunits = units;
  // partial slots: one per workgroup on the narrow MFMA paths (its four pairs
  // fold their splits first), one per split (VALU) or per pair (wide)
  const size_t nslot = pl.mfma && !pl.wide ? (size_t)wg / 4 : (size_t)wg;
  pl.off_ml = 0;
  pl.off_o = pl.off_ml + (nslot * p.rows_chunk * 2 * 4 + 255) / 256 * 256;
  pl.off_flags = pl.off_o + nslot * p.rows_chunk * p.D * 4;
  // the int8 MFMA path's per-workgroup conversion flags
  pl.ws_bytes = pl.off_flags + (pl.mfma && L->dtype == TTV_I8 ? (size_t)wg / 4 * 4 : 0);
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

extern "C" size_t tree_verify_attention_window_ws(const ttv_batch* batch, int32_t Hq, const ttv_kv_layer* layer,
                                                  int32_t q_dtype, int32_t window) {
  AttnPlan pl;
  if (window < 1 || plan_attention(batch, Hq, layer, q_dtype, pl, window) != TTV_OK) return 0;
  return pl.ws_bytes;
}

static ttv_status run_attention(const ttv_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                                const ttv_kv_layer* layer, const uint64_t* anc, float softmax_scale, int window,
                                float* out, void* ws, size_t ws_bytes, void* stream) {
  AttnPlan pl;
  ttv_status s = plan_attention(batch, Hq, layer, q_dtype, pl, window);
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
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_ml);
  p.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_o);
  p.exact_flags = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.off_flags);
  p.scale_log2 = softmax_scale * kLog2e;
  const unsigned grid = static_cast<unsigned>((p.nwg + kNumXcd - 1) / kNumXcd * kNumXcd);
  const unsigned mgrid = static_cast<unsigned>((p.nwg / 4 + kNumXcd - 1) / kNumXcd * kNumXcd);
  hipStream_t st = (hipStream_t)stream;
  const bool i8 = layer->dtype == TTV_I8;
  if (pl.mfma) {
#define TTV_MFMA(I, R0, R1) \
  hipLaunchKernelGGL((attn_bf16_narrow_kernel<R0, R1, 2>), dim3(mgrid), dim3(512), 0, st, p)
#define TTV_WIDE(R0, R1) hipLaunchKernelGGL((attn_bf16_split_kernel<kWideMaxRB>), dim3(mgrid), dim3(512), 0, st, p)
#define TTV_MFMA_RB(R0, R1) TTV_MFMA(false, R0, R1)
#define TTV_SPLIT(R)                                                                                  \
  do {                                                                                                \
    if (pl.i8_one_launch) {                                                                           \
      hipLaunchKernelGGL((attn_i8_split_kernel<R, kI8Exact>), dim3(mgrid), dim3(512), 0, st, p);       \
    } else {                                                                                          \
      hipLaunchKernelGGL((attn_i8_split_kernel<R, kI8Offset>), dim3(mgrid), dim3(512), 0, st, p);      \
      hipLaunchKernelGGL((attn_i8_split_kernel<R, kI8Flagged>), dim3(mgrid), dim3(512), 0, st, p);     \
    }                                                                                                 \
  } while (0)
    if (i8) {
      switch (pl.rb) {
        case 1: TTV_SPLIT(1); break;
        case 2: TTV_SPLIT(2); break;
        case 3: TTV_SPLIT(3); break;
        case 4: TTV_SPLIT(4); break;
        default: TTV_SPLIT(5); break;
      }
    } else if (pl.wide) {
      TTV_WIDE(2, 2);  // up to 4 row blocks per chunk; each wave runs its own count
    } else switch (pl.rb) {  // row blocks of a chunk, split between the two waves of a pair
      case 1: case 2: TTV_MFMA_RB(1, 1); break;
      case 3: TTV_MFMA_RB(2, 1); break;
      case 4: TTV_MFMA_RB(2, 2); break;
      case 5: TTV_MFMA_RB(3, 2); break;
      default: TTV_MFMA_RB(3, 3); break;
    }
#undef TTV_MFMA_RB
#undef TTV_WIDE
#undef TTV_SPLIT
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
  s = check_launch("tree_verify_attention");
  if (s != TTV_OK || !pl.merge) return s;
  hipLaunchKernelGGL(merge_kernel,
                     dim3(static_cast<unsigned>(pl.nunits), static_cast<unsigned>((p.rows_chunk + kMergeRows - 1) / kMergeRows)),
                     dim3(kMergeThreads), 0, st, p, pl.mfma && !pl.wide ? 4 : 1);
  return check_launch("tree_verify_attention merge");
}

extern "C" ttv_status tree_verify_attention(const ttv_batch* batch, const void* q, int32_t q_dtype, int32_t Hq,
                                            const ttv_kv_layer* layer, const uint64_t* anc, float softmax_scale,
                                            float* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  return run_attention(batch, q, q_dtype, Hq, layer, anc, softmax_scale, 0, out, ws, ws_bytes, stream);
}

// ------------------------------------------------ allocation-free form ----
// tree_verify_attention_static keeps the partials in this file-scope device
// array instead of a caller workspace. Every device that runs the library
// holds its own copy until the process ends. In host code the array's name
// is only a stand-in: the per-device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// passed to kernels.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device: the address of its scratch copy
}  // namespace

// The scratch address on the device `stream` runs on (the current device for
// the NULL stream); looked up on the first call for that device.
static ttv_status static_scratch(void* stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  TTV_REQUIRE(e == hipSuccess, TTV_ERR_HIP, "tree_verify_attention_static: no current device: %s",
              hipGetErrorString(e));
  dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    TTV_REQUIRE(e == hipSuccess, TTV_ERR_HIP, "tree_verify_attention_static: stream device: %s",
                hipGetErrorString(e));
  }
  TTV_REQUIRE(dev >= 0 && dev < kMaxDevices, TTV_ERR_UNSUPPORTED,
              "tree_verify_attention_static: device %d is beyond the %d devices the scratch table holds", dev,
              kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur) {
      e = hipSetDevice(dev);
      TTV_REQUIRE(e == hipSuccess, TTV_ERR_HIP, "tree_verify_attention_static: hipSetDevice(%d): %s", dev,
                  hipGetErrorString(e));
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    TTV_REQUIRE(e == hipSuccess && ptr != nullptr, TTV_ERR_HIP,
                "tree_verify_attention_static: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TTV_OK;
}

extern "C" ttv_status tree_verify_attention_static(const ttv_batch* batch, const void* q, int32_t q_dtype,
                                                   int32_t Hq, const ttv_kv_layer* layer, const uint64_t* anc,
                                                   float softmax_scale, float* out, void* stream) {
  clear_error();
  AttnPlan pl;
  ttv_status s = plan_attention(batch, Hq, layer, q_dtype, pl);
  if (s != TTV_OK) return s;
  TTV_REQUIRE(pl.ws_bytes <= kStaticScratchBytes, TTV_ERR_UNSUPPORTED,
              "tree_verify_attention_static: the call needs %zu bytes of partials, the static scratch holds %zu "
              "(tree_verify_attention takes a workspace of any size)", pl.ws_bytes, kStaticScratchBytes);
  if (pl.prm.nwg == 0) return TTV_OK;
  void* ws = nullptr;
  s = static_scratch(stream, &ws);
  if (s != TTV_OK) return s;
  return run_attention(batch, q, q_dtype, Hq, layer, anc, softmax_scale, 0, out, ws, kStaticScratchBytes, stream);
}

extern "C" ttv_status tree_verify_attention_window(const ttv_batch* batch, const void* q, int32_t q_dtype,
                                                   int32_t Hq, const ttv_kv_layer* layer, const uint64_t* anc,
                                                   float softmax_scale, int32_t window, float* out, void* ws,
                                                   size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(window >= 1, TTV_ERR_INVALID, "tree_verify_attention_window: window %d < 1", window);
  return run_attention(batch, q, q_dtype, Hq, layer, anc, softmax_scale, window, out, ws, ws_bytes, stream);
}
