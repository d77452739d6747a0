// Step 5 of a verify round: rollback by gather along the sequence axis.
//
// [I1204] mlxcel issue #1204, "The rollback constraint, which decides
// feasibility": a chain's accepted set is a prefix (a tail trim suffices); a
// tree's accepted path is scattered across the block, so the survivors are
// selected and compacted. [PR1212] mlxcel PR #1212: the gather_positions
// commit (select and close up a scattered set; int8 scale sidecars move with
// their tokens; a prefix selection equals trim_to; the identity selection
// moves nothing), the commit widening it to every sequence-axis buffer, and
// the gather_within_tail commit (rewrite only the part of the window that
// changes, so the cost follows the block rather than the context).
//
// Launch sequence for one call:
//  1. validate: workgroups over (chunk, sequence) check the selection
//     (strictly increasing, in range, not longer than the live window or the
//     row stride); a one-workgroup pass folds the chunks into j0, the first j
//     with sel[j] != j, and a bad flag per sequence.
//  2. copy: every workgroup first checks all sequences' bad flags (one wave
//     load + ballot) and leaves without writing if any is set, so a malformed
//     call writes nothing at all.
//     - out of place: one workgroup per (layer, sequence, head, 256-row chunk)
//       streams 16-byte pieces of K and V rows plus the scale sidecars.
//     - in place: one workgroup per (layer, sequence, head) moves rows
//       j >= j0 in ascending chunks. Sources satisfy sel[j] > j there, so a
//       chunk only overwrites rows below every later chunk's sources; inside a
//       chunk all reads complete (barrier) before any write.
#include "common.hpp"

namespace ttv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
static_assert(kMaxGatherRowBytes == 16 * kGatherThreads, "one row per pass of 16-byte pieces");
constexpr int kLayersPerLaunch = 16;
constexpr int kTakeRows = 512;  // rows per out-of-place workgroup
constexpr int kMaxSelChunks = 64;     // validation workgroups per sequence, at most
constexpr int kMinSelChunk = 2048;    // selection entries per validation workgroup, at least

struct LayerPtrs {
  const char* k[kLayersPerLaunch];
  const char* v[kLayersPerLaunch];
  const uint16_t* ks[kLayersPerLaunch];
  const uint16_t* vs[kLayersPerLaunch];
  char* dk[kLayersPerLaunch];
  char* dv[kLayersPerLaunch];
  uint16_t* dks[kLayersPerLaunch];
  uint16_t* dvs[kLayersPerLaunch];
};

struct LiveLens {
  int32_t live[TTV_MAX_BATCH];
};

// One workgroup per (chunk of the selection, sequence): partial j0 and bad flag.
__global__ void __launch_bounds__(kGatherThreads) sel_validate_kernel(const int32_t* __restrict__ sel,
                                                                      int sel_stride,
                                                                      const int32_t* __restrict__ sel_len,
                                                                      LiveLens lens, int chunk,
                                                                      int32_t* __restrict__ part_j0,
                                                                      int32_t* __restrict__ part_bad) {
  __shared__ int s_j0;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int n = sel_len[b];
  const int live = lens.live[b];
  if (threadIdx.x == 0) s_j0 = n;
  __syncthreads();
  int bad = (n < 0 || n > live || n > sel_stride) ? 1 : 0;
  if (!bad) {
    const int32_t* row = sel + static_cast<int64_t>(b) * sel_stride;
    const int j1 = (c + 1) * chunk < n ? (c + 1) * chunk : n;
    int j0 = n;
    for (int j = c * chunk + threadIdx.x; j < j1; j += kGatherThreads) {
      const int s = row[j];
      if (s < 0 || s >= live) bad = 1;
      if (j + 1 < n && row[j + 1] <= s) bad = 1;
      if (s != j && j < j0) j0 = j;
    }
    if (j0 < n) atomicMin(&s_j0, j0);
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    part_j0[b * kMaxSelChunks + c] = s_j0;
    part_bad[b * kMaxSelChunks + c] = bad;
  }
}

// One thread per sequence folds the chunk partials into j0[b] and bad[b].
__global__ void __launch_bounds__(TTV_MAX_BATCH) sel_finalize_kernel(const int32_t* __restrict__ part_j0,
                                                                     const int32_t* __restrict__ part_bad,
                                                                     int B, int nch, int32_t* __restrict__ j0_out,
                                                                     int32_t* __restrict__ bad_out,
                                                                     int32_t* __restrict__ status) {
  const int b = threadIdx.x;
  if (b >= B) return;
  int j0 = 0x7FFFFFFF, bad = 0;
  for (int c = 0; c < nch; ++c) {
    const int v = part_j0[b * kMaxSelChunks + c];
    j0 = v < j0 ? v : j0;
    bad |= part_bad[b * kMaxSelChunks + c];
  }
  j0_out[b] = j0;
  bad_out[b] = bad;
  if (bad) *status = TTV_DEV_BAD_SELECTION;
}

// Tail form: per sequence b, the tail starts at row start[b] and holds len[b]
// (<= 64) rows; kept offsets index into it.
struct TailSpec {
  int32_t start[TTV_MAX_BATCH];
  int32_t len[TTV_MAX_BATCH];
};

// One wave per sequence checks the kept offsets (at most 64, one per lane):
// strictly increasing, inside the tail, no more than the tail or the row
// stride holds. Writes j0 (absolute first moved row), the absolute end
// start + kept_len, the tail start and a bad flag per sequence.
__global__ void __launch_bounds__(kWave) tail_validate_kernel(const int32_t* __restrict__ kept, int kept_stride,
                                                              const int32_t* __restrict__ kept_len, TailSpec tails,
                                                              int32_t* __restrict__ j0s, int32_t* __restrict__ ends,
                                                              int32_t* __restrict__ starts,
                                                              int32_t* __restrict__ bad_out,
                                                              int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int ts = tails.start[b];
  const int tl = tails.len[b];
  const int n = kept_len[b];
  int f = (n < 0 || n > tl || n > kept_stride) ? 1 : 0;
  int k = lane;
  if (!f && lane < n) {
    const int32_t* __restrict__ row = kept + static_cast<int64_t>(b) * kept_stride;
    k = row[lane];
    if (k < 0 || k >= tl) f = 1;
    if (lane + 1 < n && row[lane + 1] <= k) f = 1;
  }
  const bool any = __ballot(f != 0) != 0;
  const uint64_t moved = __ballot(lane < n && k != lane);
  if (lane == 0) {
    const int nn = any ? 0 : n;
    const int j = (!any && moved != 0) ? __builtin_ctzll(moved) : nn;
    j0s[b] = ts + j;
    ends[b] = ts + nn;
    starts[b] = ts;
    bad_out[b] = any ? 1 : 0;
    if (any) *status = TTV_DEV_BAD_SELECTION;
  }
}

__device__ __forceinline__ bool any_bad(const int32_t* __restrict__ bad, int B) {
  // wave 0 of the block reads all flags; the answer is shared through LDS
  __shared__ int s_bad;
  if (threadIdx.x < kWave) {
    int f = 0;
    for (int b = threadIdx.x; b < B; b += kWave) f |= bad[b];
    const uint64_t m = __ballot(f != 0);
    if (threadIdx.x == 0) s_bad = m != 0;
  }
  __syncthreads();
  return s_bad != 0;
}

// Out-of-place take: dst rows [0, n) <- src rows sel[0..n).
__global__ void __launch_bounds__(kGatherThreads) take_kernel(LayerPtrs L, int B, int Hkv, int cap, int row_bytes,
                                                              int chunks_per_head, const int32_t* __restrict__ sel,
                                                              int sel_stride, const int32_t* __restrict__ sel_len,
                                                              const int32_t* __restrict__ bad) {
  if (any_bad(bad, B)) return;
  int w = blockIdx.x;
  const int chunk = w % chunks_per_head;
  w /= chunks_per_head;
  const int h = w % Hkv;
  w /= Hkv;
  const int b = w % B;
  const int l = w / B;
  const int n = sel_len[b];
  const int r0 = chunk * kTakeRows;
  if (r0 >= n) return;
  const int r1 = r0 + kTakeRows < n ? r0 + kTakeRows : n;
  const int32_t* __restrict__ srow = sel + static_cast<int64_t>(b) * sel_stride;
  const int64_t head = static_cast<int64_t>(b) * Hkv + h;
  const int64_t base = head * cap;
  const int U = row_bytes >> 4;  // 16-byte pieces per row
  const int rows_per_pass = kGatherThreads / U;
  const int u = threadIdx.x % U;
  const int rr = threadIdx.x / U;
  const bool copier = rr < rows_per_pass;
  const char* __restrict__ ks = L.k[l];
  const char* __restrict__ vs = L.v[l];
  char* __restrict__ kd = L.dk[l];
  char* __restrict__ vd = L.dv[l];
  // batches of kTakeBatch passes: every index, then every K/V piece of the
  // batch in flight before the first store (a thread keeps up to 2 x 16 x 16
  // bytes moving instead of 2 x 16)
  constexpr int kTakeBatch = 16;
  for (int jb = r0 + rr; copier && jb < r1; jb += kTakeBatch * rows_per_pass) {
    int sj[kTakeBatch];
#pragma unroll
    for (int q = 0; q < kTakeBatch; ++q) {
      const int j = jb + q * rows_per_pass;
      sj[q] = j < r1 ? srow[j] : 0;
    }
    u32x4 a[kTakeBatch], c[kTakeBatch];
#pragma unroll
    for (int q = 0; q < kTakeBatch; ++q) {
      if (jb + q * rows_per_pass < r1) {
        const int64_t src = (base + sj[q]) * row_bytes + 16 * u;
        a[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + src));
        c[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + src));
      }
    }
#pragma unroll
    for (int q = 0; q < kTakeBatch; ++q) {
      const int j = jb + q * rows_per_pass;
      if (j < r1) {
        const int64_t dst = (base + j) * row_bytes + 16 * u;
        __builtin_nontemporal_store(a[q], reinterpret_cast<u32x4*>(kd + dst));
        __builtin_nontemporal_store(c[q], reinterpret_cast<u32x4*>(vd + dst));
      }
    }
  }
  if (L.ks[l] != nullptr) {
    for (int j = r0 + threadIdx.x; j < r1; j += kGatherThreads) {
      const int s = srow[j];
      L.dks[l][base + j] = L.ks[l][base + s];
      L.dvs[l][base + j] = L.vs[l][base + s];
    }
  }
}

// In-place compaction of rows j >= j0 for one (layer, sequence, head).
// Absolute selection (TAIL = false): row j <- row sel[b][j], j < sel_len[b].
// Tail form (TAIL = true): sel[b] holds offsets inside the tail that starts at
// row tail_start[b], row tail_start + j <- row tail_start + sel[b][j], and
// sel_len[b] is the absolute end tail_start + kept_len.
template <int PIECES, bool TAIL>  // PIECES: 16-byte pieces of K (and of V) held per thread per chunk
__global__ void __launch_bounds__(kGatherThreads) compact_kernel(LayerPtrs L, int B, int Hkv, int cap, int row_bytes,
                                                                 const int32_t* __restrict__ sel, int sel_stride,
                                                                 const int32_t* __restrict__ sel_len,
                                                                 const int32_t* __restrict__ j0s,
                                                                 const int32_t* __restrict__ bad,
                                                                 const int32_t* __restrict__ tail_start) {
  if (any_bad(bad, B)) return;
  int w = blockIdx.x;
  const int h = w % Hkv;
  w /= Hkv;
  const int b = w % B;
  const int l = w / B;
  const int n = sel_len[b];
  const int j0 = j0s[b];
  if (j0 >= n) return;  // identity or prefix selection: nothing moves
  const int32_t* __restrict__ srow = sel + static_cast<int64_t>(b) * sel_stride;
  const int ts = TAIL ? tail_start[b] : 0;
  const int64_t base = (static_cast<int64_t>(b) * Hkv + h) * cap;
  const int U = row_bytes >> 4;  // <= kGatherThreads (kv_can_gather), so a chunk holds >= PIECES rows
  const int rows_chunk = PIECES * kGatherThreads / U < kGatherThreads ? PIECES * kGatherThreads / U : kGatherThreads;
  char* __restrict__ kp = const_cast<char*>(L.k[l]);
  char* __restrict__ vp = const_cast<char*>(L.v[l]);
  uint16_t* __restrict__ ksp = const_cast<uint16_t*>(L.ks[l]);
  uint16_t* __restrict__ vsp = const_cast<uint16_t*>(L.vs[l]);
  for (int c0 = j0; c0 < n; c0 += rows_chunk) {
    const int c1 = c0 + rows_chunk < n ? c0 + rows_chunk : n;
    u32x4 kr[PIECES], vr[PIECES];
    uint16_t ksr = 0, vsr = 0;
#pragma unroll
    for (int p = 0; p < PIECES; ++p) {
      const int q = threadIdx.x + p * kGatherThreads;  // piece id within the chunk
      const int j = c0 + q / U;
      if (j < c1) {
        const int64_t src = (base + ts + srow[j - ts]) * row_bytes + 16 * (q % U);
        kr[p] = *reinterpret_cast<const u32x4*>(kp + src);
        vr[p] = *reinterpret_cast<const u32x4*>(vp + src);
      }
    }
    const int js = c0 + threadIdx.x;
    if (ksp != nullptr && threadIdx.x < rows_chunk && js < c1) {
      ksr = ksp[base + ts + srow[js - ts]];
      vsr = vsp[base + ts + srow[js - ts]];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PIECES; ++p) {
      const int q = threadIdx.x + p * kGatherThreads;
      const int j = c0 + q / U;
      if (j < c1) {
        const int64_t dst = (base + j) * row_bytes + 16 * (q % U);
        *reinterpret_cast<u32x4*>(kp + dst) = kr[p];
        *reinterpret_cast<u32x4*>(vp + dst) = vr[p];
      }
    }
    if (ksp != nullptr && threadIdx.x < rows_chunk && js < c1) {
      ksp[base + js] = ksr;
      vsp[base + js] = vsr;
    }
    __syncthreads();
  }
}

static bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace ttv

using namespace ttv;

extern "C" size_t kv_gather_positions_ws(int32_t B) {
  if (B <= 0) return 0;
  return (2 + 2 * static_cast<size_t>(kMaxSelChunks)) * static_cast<size_t>(B) * sizeof(int32_t);
}

extern "C" ttv_status kv_gather_positions(const ttv_kv_layer* src, const ttv_kv_layer* dst, int32_t n_layers,
                                          int32_t B, const int32_t* sel, int32_t sel_stride,
                                          const int32_t* sel_len, const int32_t* live_len_h,
                                          int32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(n_layers >= 0 && B >= 0 && B <= TTV_MAX_BATCH, TTV_ERR_INVALID,
              "kv_gather_positions: n_layers %d, B %d", n_layers, B);
  if (n_layers == 0 || B == 0) return TTV_OK;
  ttv_status cap_ok = kv_can_gather(src, n_layers);
  if (cap_ok != TTV_OK) return cap_ok;
  TTV_REQUIRE(sel && sel_len && live_len_h && dev_status, TTV_ERR_INVALID, "kv_gather_positions: NULL pointer");
  TTV_REQUIRE(sel_stride >= 0, TTV_ERR_INVALID, "kv_gather_positions: negative sel_stride");
  const size_t need = kv_gather_positions_ws(B);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "kv_gather_positions: workspace %zu bytes < %zu",
              ws_bytes, need);
  const ttv_kv_layer& L0 = src[0];
  int max_live = 0;
  for (int b = 0; b < B; ++b) {
    TTV_REQUIRE(live_len_h[b] >= 0 && live_len_h[b] <= L0.cap, TTV_ERR_INVALID,
                "kv_gather_positions: live_len[%d] = %d outside [0, cap %d]", b, live_len_h[b], L0.cap);
    max_live = live_len_h[b] > max_live ? live_len_h[b] : max_live;
  }
  bool in_place = true;
  for (int l = 0; l < n_layers; ++l) {
    const ttv_kv_layer& s = src[l];
    TTV_REQUIRE(s.dtype == L0.dtype && s.Hkv == L0.Hkv && s.D == L0.D && s.cap == L0.cap, TTV_ERR_INVALID,
                "kv_gather_positions: layer %d shape/dtype differs from layer 0", l);
    if (dst != nullptr) {
      const ttv_kv_layer& d = dst[l];
      TTV_REQUIRE(d.dtype == s.dtype && d.Hkv == s.Hkv && d.D == s.D && d.cap == s.cap, TTV_ERR_INVALID,
                  "kv_gather_positions: dst layer %d shape/dtype differs from src", l);
      const bool same = d.k == s.k && d.v == s.v && d.k_scale == s.k_scale && d.v_scale == s.v_scale;
      if (!same) in_place = false;
    }
  }
  const int esz = L0.dtype == TTV_F32 ? 4 : L0.dtype == TTV_BF16 ? 2 : 1;
  const int row_bytes = L0.D * esz;
  const size_t kv_bytes = static_cast<size_t>(B) * L0.Hkv * L0.cap * row_bytes;
  const size_t sc_bytes = static_cast<size_t>(B) * L0.Hkv * L0.cap * 2;
  if (!in_place) {
    for (int l = 0; l < n_layers; ++l) {
      const ttv_kv_layer& s = src[l];
      const ttv_kv_layer& d = dst[l];
      TTV_REQUIRE(d.k && d.v && (d.dtype != TTV_I8 || (d.k_scale && d.v_scale)), TTV_ERR_INVALID,
                  "kv_gather_positions: dst layer %d is missing a buffer", l);
      for (int a = 0; a < n_layers; ++a) {
        const ttv_kv_layer& t = src[a];
        const bool ov = ranges_overlap(d.k, kv_bytes, t.k, kv_bytes) || ranges_overlap(d.k, kv_bytes, t.v, kv_bytes) ||
                        ranges_overlap(d.v, kv_bytes, t.k, kv_bytes) || ranges_overlap(d.v, kv_bytes, t.v, kv_bytes) ||
                        (s.dtype == TTV_I8 &&
                         (ranges_overlap(d.k_scale, sc_bytes, t.k_scale, sc_bytes) ||
                          ranges_overlap(d.k_scale, sc_bytes, t.v_scale, sc_bytes) ||
                          ranges_overlap(d.v_scale, sc_bytes, t.k_scale, sc_bytes) ||
                          ranges_overlap(d.v_scale, sc_bytes, t.v_scale, sc_bytes)));
        TTV_REQUIRE(!ov, TTV_ERR_INVALID,
                    "kv_gather_positions: dst layer %d overlaps src layer %d (only exact in-place aliasing "
                    "is allowed)", l, a);
      }
    }
  }
  int32_t* j0s = static_cast<int32_t*>(ws);
  int32_t* bad = j0s + B;
  int32_t* part_j0 = bad + B;
  int32_t* part_bad = part_j0 + static_cast<size_t>(B) * kMaxSelChunks;
  // a valid selection is no longer than the live window or the row stride
  const int max_n = max_live < sel_stride ? max_live : sel_stride;
  int chunk = (max_n + kMaxSelChunks - 1) / kMaxSelChunks;
  chunk = chunk < kMinSelChunk ? kMinSelChunk : (chunk + 255) / 256 * 256;
  const int nch = max_n == 0 ? 1 : (max_n + chunk - 1) / chunk;
  // the largest copy grid (a launch of kLayersPerLaunch layers), checked before anything is launched
  const int take_chunks = (max_live + kTakeRows - 1) / kTakeRows;
  const int64_t max_grid = static_cast<int64_t>(n_layers < kLayersPerLaunch ? n_layers : kLayersPerLaunch) * B *
                           L0.Hkv * (in_place ? 1 : take_chunks);
  TTV_REQUIRE(max_grid <= 0x7FFFFFFF, TTV_ERR_INVALID, "kv_gather_positions: grid too large");
  hipStream_t st = (hipStream_t)stream;
  LiveLens lens{};
  for (int b = 0; b < B; ++b) lens.live[b] = live_len_h[b];
  hipLaunchKernelGGL(sel_validate_kernel, dim3(nch, B), dim3(kGatherThreads), 0, st, sel, sel_stride, sel_len,
                     lens, chunk, part_j0, part_bad);
  hipLaunchKernelGGL(sel_finalize_kernel, dim3(1), dim3(TTV_MAX_BATCH), 0, st, part_j0, part_bad, B, nch, j0s, bad,
                     dev_status);
  ttv_status s = check_launch("kv_gather_positions validate");
  if (s != TTV_OK) return s;
  for (int l0 = 0; l0 < n_layers; l0 += kLayersPerLaunch) {
    const int nl = n_layers - l0 < kLayersPerLaunch ? n_layers - l0 : kLayersPerLaunch;
    LayerPtrs P{};
    for (int i = 0; i < nl; ++i) {
      const ttv_kv_layer& a = src[l0 + i];
      const ttv_kv_layer& d = in_place ? a : dst[l0 + i];
      P.k[i] = static_cast<const char*>(a.k);
      P.v[i] = static_cast<const char*>(a.v);
      P.ks[i] = a.dtype == TTV_I8 ? a.k_scale : nullptr;
      P.vs[i] = a.dtype == TTV_I8 ? a.v_scale : nullptr;
      P.dk[i] = static_cast<char*>(d.k);
      P.dv[i] = static_cast<char*>(d.v);
      P.dks[i] = a.dtype == TTV_I8 ? d.k_scale : nullptr;
      P.dvs[i] = a.dtype == TTV_I8 ? d.v_scale : nullptr;
    }
    if (in_place) {
      const int64_t nblk = static_cast<int64_t>(nl) * B * L0.Hkv;  // <= max_grid
      // at most 4 pieces of 16 B per buffer per thread: 1024 rows of int8 D=64 ... 32 rows of f32 D=512
      hipLaunchKernelGGL((compact_kernel<4, false>), dim3(static_cast<unsigned>(nblk)), dim3(kGatherThreads), 0, st, P,
                         B, L0.Hkv, L0.cap, row_bytes, sel, sel_stride, sel_len, j0s, bad, nullptr);
    } else {
      const int chunks = take_chunks;
      if (chunks == 0) continue;
      const int64_t nblk = static_cast<int64_t>(nl) * B * L0.Hkv * chunks;  // <= max_grid
      hipLaunchKernelGGL(take_kernel, dim3(static_cast<unsigned>(nblk)), dim3(kGatherThreads), 0, st, P, B, L0.Hkv,
                         L0.cap, row_bytes, chunks, sel, sel_stride, sel_len, bad);
    }
    s = check_launch("kv_gather_positions copy");
    if (s != TTV_OK) return s;
  }
  return TTV_OK;
}

extern "C" ttv_status kv_can_gather_within_tail(const ttv_kv_layer* layers, int32_t n_layers, int32_t B,
                                                const int32_t* ring_wrapped_h) {
  clear_error();
  TTV_REQUIRE(B >= 0 && B <= TTV_MAX_BATCH, TTV_ERR_INVALID, "kv_can_gather_within_tail: B %d", B);
  ttv_status s = kv_can_gather(layers, n_layers);
  if (s != TTV_OK) return s;
  if (ring_wrapped_h != nullptr)
    for (int b = 0; b < B; ++b)
      TTV_REQUIRE(ring_wrapped_h[b] == 0, TTV_ERR_UNSUPPORTED,
                  "kv_gather_within_tail: the rotating cache of sequence %d has wrapped, so its tail is no longer "
                  "in logical order", b);
  return TTV_OK;
}

extern "C" size_t kv_gather_within_tail_ws(int32_t B) {
  if (B <= 0) return 0;
  return 4 * static_cast<size_t>(B) * sizeof(int32_t);
}

extern "C" ttv_status kv_gather_within_tail(const ttv_kv_layer* layers, int32_t n_layers, int32_t B,
                                            const int32_t* kept, int32_t kept_stride, const int32_t* kept_len,
                                            const int32_t* live_len_h, const int32_t* tail_len_h,
                                            const int32_t* ring_wrapped_h, int32_t* dev_status, void* ws,
                                            size_t ws_bytes, void* stream) {
  clear_error();
  TTV_REQUIRE(n_layers >= 0 && B >= 0 && B <= TTV_MAX_BATCH, TTV_ERR_INVALID,
              "kv_gather_within_tail: n_layers %d, B %d", n_layers, B);
  if (n_layers == 0 || B == 0) return TTV_OK;
  ttv_status s = kv_can_gather_within_tail(layers, n_layers, B, ring_wrapped_h);
  if (s != TTV_OK) return s;
  TTV_REQUIRE(kept && kept_len && live_len_h && tail_len_h && dev_status, TTV_ERR_INVALID,
              "kv_gather_within_tail: NULL pointer");
  TTV_REQUIRE(kept_stride >= 0, TTV_ERR_INVALID, "kv_gather_within_tail: negative kept_stride");
  const size_t need = kv_gather_within_tail_ws(B);
  TTV_REQUIRE(ws && ws_bytes >= need, TTV_ERR_WORKSPACE, "kv_gather_within_tail: workspace %zu bytes < %zu",
              ws_bytes, need);
  const ttv_kv_layer& L0 = layers[0];
  for (int l = 0; l < n_layers; ++l) {
    const ttv_kv_layer& a = layers[l];
    TTV_REQUIRE(a.dtype == L0.dtype && a.Hkv == L0.Hkv && a.D == L0.D && a.cap == L0.cap, TTV_ERR_INVALID,
                "kv_gather_within_tail: layer %d shape/dtype differs from layer 0", l);
  }
  TailSpec tails{};
  for (int b = 0; b < B; ++b) {
    const int live = live_len_h[b], tl = tail_len_h[b];
    TTV_REQUIRE(live >= 0 && live <= L0.cap, TTV_ERR_INVALID,
                "kv_gather_within_tail: live_len[%d] = %d outside [0, cap %d]", b, live, L0.cap);
    TTV_REQUIRE(tl >= 0 && tl <= live && tl <= TTV_MAX_NODES, TTV_ERR_INVALID,
                "kv_gather_within_tail: tail_len[%d] = %d outside [0, min(live_len %d, %d)]", b, tl, live,
                TTV_MAX_NODES);
    tails.start[b] = live - tl;
    tails.len[b] = tl;
  }
  const int esz = L0.dtype == TTV_F32 ? 4 : L0.dtype == TTV_BF16 ? 2 : 1;
  const int row_bytes = L0.D * esz;
  int32_t* j0s = static_cast<int32_t*>(ws);
  int32_t* ends = j0s + B;
  int32_t* starts = ends + B;
  int32_t* bad = starts + B;
  TTV_REQUIRE(static_cast<int64_t>(n_layers < kLayersPerLaunch ? n_layers : kLayersPerLaunch) * B * L0.Hkv <=
                  0x7FFFFFFF,
              TTV_ERR_INVALID, "kv_gather_within_tail: grid too large");
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(tail_validate_kernel, dim3(B), dim3(kWave), 0, st, kept, kept_stride, kept_len, tails, j0s,
                     ends, starts, bad, dev_status);
  s = check_launch("kv_gather_within_tail validate");
  if (s != TTV_OK) return s;
  for (int l0 = 0; l0 < n_layers; l0 += kLayersPerLaunch) {
    const int nl = n_layers - l0 < kLayersPerLaunch ? n_layers - l0 : kLayersPerLaunch;
    LayerPtrs P{};
    for (int i = 0; i < nl; ++i) {
      const ttv_kv_layer& a = layers[l0 + i];
      P.k[i] = static_cast<const char*>(a.k);
      P.v[i] = static_cast<const char*>(a.v);
      P.ks[i] = a.dtype == TTV_I8 ? a.k_scale : nullptr;
      P.vs[i] = a.dtype == TTV_I8 ? a.v_scale : nullptr;
      P.dk[i] = static_cast<char*>(a.k);
      P.dv[i] = static_cast<char*>(a.v);
      P.dks[i] = P.ks[i] ? a.k_scale : nullptr;
      P.dvs[i] = P.vs[i] ? a.v_scale : nullptr;
    }
    const int64_t nblk = static_cast<int64_t>(nl) * B * L0.Hkv;  // checked above
    hipLaunchKernelGGL((compact_kernel<4, true>), dim3(static_cast<unsigned>(nblk)), dim3(kGatherThreads), 0, st, P,
                       B, L0.Hkv, L0.cap, row_bytes, kept, kept_stride, ends, j0s, bad, starts);
    s = check_launch("kv_gather_within_tail copy");
    if (s != TTV_OK) return s;
  }
  return TTV_OK;
}
