// Steps 1 and 4 of a verify round -- the ancestor mask and the accept walk --
// plus the error plumbing and the capability query. One wavefront owns one
// draft tree (T <= 64 = wave width): lane i holds node i.
//
// Sources: [I1204] mlxcel issue #1204 "draft a tree instead of a chain",
// sections "What this needs", "Increment 1 ... topology, mask, walk",
// "Increment 3: the mask is now the shape a forward actually takes";
// [PR1212] mlxcel PR #1212, history-mask, rollback-to-path and
// tree_round_is_available commits; [S728] splash issue #728 "What it does".
#include "common.hpp"

#include <string>

namespace ttv {

static thread_local std::string g_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
}

void clear_error() { g_error.clear(); }

ttv_status check_batch(const ttv_batch* batch, bool need_device) {
  TTV_REQUIRE(batch != nullptr, TTV_ERR_INVALID, "batch is NULL");
  const int B = batch->B;
  TTV_REQUIRE(B >= 0 && B <= TTV_MAX_BATCH, TTV_ERR_INVALID, "batch size %d outside [0, %d]", B,
              TTV_MAX_BATCH);
  if (B == 0) return TTV_OK;
  TTV_REQUIRE(batch->node_off_h && batch->hist_len_h, TTV_ERR_INVALID, "host node_off/hist_len missing");
  if (need_device)
    TTV_REQUIRE(batch->node_off_d && batch->hist_len_d, TTV_ERR_INVALID,
                "device node_off/hist_len missing");
  TTV_REQUIRE(batch->node_off_h[0] == 0, TTV_ERR_INVALID, "node_off[0] must be 0");
  for (int b = 0; b < B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    TTV_REQUIRE(T >= 0 && T <= TTV_MAX_NODES, TTV_ERR_INVALID,
                "sequence %d has %d nodes; a tree holds 0..%d", b, T, TTV_MAX_NODES);
    TTV_REQUIRE(batch->hist_len_h[b] >= 0, TTV_ERR_INVALID, "hist_len[%d] < 0", b);
  }
  return TTV_OK;
}

// ------------------------------------------------------------------ mask ----
// anc(i) = {i} U anc(parent(i)). Pointer jumping: A_i starts as {i} and J_i as
// parent(i); each round A_i |= A_{J_i}, J_i = J_{J_i}, so after r rounds A_i
// holds the 2^r nearest nodes of i's root path; 6 rounds cover depth 63.
__global__ void __launch_bounds__(64) mask_kernel(const int32_t* __restrict__ node_off,
                                                  const int32_t* __restrict__ parent,
                                                  uint64_t* __restrict__ anc,
                                                  int32_t* __restrict__ depth,
                                                  int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int o0 = node_off[b];
  const int T = node_off[b + 1] - o0;
  if (T <= 0) return;
  const bool active = lane < T;
  const int p = active ? parent[o0 + lane] : -1;
  const bool ok = !active || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  if (__ballot(!ok) != 0) {
    if (lane == 0) *status = TTV_DEV_BAD_PARENT;
    return;
  }
  uint64_t A = active ? (1ull << lane) : 0ull;
  int J = p;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = J < 0 ? lane : J;
    const uint64_t AJ = __shfl(A, src);
    const int JJ = __shfl(J, src);
    if (J >= 0) {
      A |= AJ;
      J = JJ;
    }
  }
  if (active) {
    anc[o0 + lane] = A;
    if (depth) depth[o0 + lane] = __popcll(A) - 1;
  }
}

__global__ void expand_kernel(const uint64_t* __restrict__ anc, int P, int T, float masked,
                              float* __restrict__ out) {
  const int i = blockIdx.y;
  const int W = P + T;
  const uint64_t a = anc[i];
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < W; c += gridDim.x * blockDim.x) {
    const bool open = c < P || ((a >> (c - P)) & 1ull);
    out[(size_t)i * W + c] = open ? 0.0f : masked;
  }
}

// Sliding-window layers' form of a caller mask ([PR1212] the commit that
// intersects the caller mask with the sliding band, and the commit stating its
// properties): query row q sits at cache position offset + q and keeps column
// c only when offset + q - window < c <= offset + q. Additive masks intersect
// by elementwise minimum, so an open band entry is 0 and a blocked one is
// `masked`; a NaN in either operand comes through as in numpy.minimum.
__global__ void band_kernel(const float* caller, int S, int offset, int window, float masked, float* out) {
  const int q = blockIdx.y;
  const int pos = offset + q;
  const float* __restrict__ src = caller + (size_t)q * S;
  float* __restrict__ dst = out + (size_t)q * S;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < S; c += gridDim.x * blockDim.x) {
    const float m = src[c];
    const float b = (c > pos - window && c <= pos) ? 0.0f : masked;
    dst[c] = (m < b || m != m) ? m : b;
  }
}

__global__ void copy_rows_kernel(const float* caller, int S, float* out) {
  const int q = blockIdx.y;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < S; c += gridDim.x * blockDim.x)
    out[(size_t)q * S + c] = caller[(size_t)q * S + c];
}

// ------------------------------------------------------------------ walk ----
// Wave 0 walks the tree: ballot over lanes whose parent is the current node
// and whose token equals the target's selection there; the lowest set bit is
// the lowest-labelled matching child. Every step moves to a larger label, so
// the loop ends within T - 1 steps. All 256 threads then write the rollback
// selection [0, P) ++ (P + path).
constexpr int kWalkPrefixChunk = 256 * 16;  // identity-prefix entries per prefix workgroup

// parent[] of one tree is a rooted topological labelling (one wave, lane = node)
__device__ __forceinline__ bool walk_tree_ok(const int32_t* __restrict__ parent, int o0, int T, int lane) {
  const bool active = lane < T;
  const int p = active ? parent[o0 + lane] : -2;
  const bool ok = !active || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  return __ballot(!ok) == 0 && T > 0;
}

// Grid (1 + prefix chunks, B). Workgroup x = 0 of sequence b walks its tree
// and writes the path, the emitted tokens and the selection's block part
// sel[P + k] = P + path[k]; workgroups x >= 1 write the identity prefix
// sel[j] = j over their chunk of [0, P), so a long history is written by many
// workgroups at once. Every workgroup checks the tree first: an invalid tree
// writes nothing.
__global__ void __launch_bounds__(256) walk_kernel(
    const int32_t* __restrict__ node_off, const int32_t* __restrict__ hist_len,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ token,
    const int32_t* __restrict__ target, int32_t* __restrict__ path, int32_t* __restrict__ path_len,
    int32_t* __restrict__ emitted, int32_t* __restrict__ sel, int sel_stride,
    int32_t* __restrict__ sel_len_out, int32_t* __restrict__ status) {
  __shared__ int s_path[TTV_MAX_NODES];
  __shared__ int s_len;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int o0 = node_off[b];
  const int T = node_off[b + 1] - o0;
  if (blockIdx.x > 0) {  // identity prefix chunk (only launched with sel)
    const int P = hist_len[b];
    const int j0 = (blockIdx.x - 1) * kWalkPrefixChunk;
    if (j0 >= P) return;  // whole workgroup
    if (tid < kWave) {
      const bool ok = walk_tree_ok(parent, o0, T, tid);
      if (tid == 0) s_len = ok ? 1 : -1;
    }
    __syncthreads();
    if (s_len < 0) return;
    int32_t* row = sel + (size_t)b * sel_stride;
    const int j1 = min(P, j0 + kWalkPrefixChunk);
    for (int j = j0 + tid; j < j1; j += blockDim.x) row[j] = j;
    return;
  }
  if (tid < kWave) {
    const int lane = tid;
    const bool active = lane < T;
    const int p = active ? parent[o0 + lane] : -2;
    const int tok = active ? token[o0 + lane] : 0;
    const bool bad = !walk_tree_ok(parent, o0, T, lane);
    int len = 0;
    if (!bad) {
      int cur = 0;
      int mine = 0;  // lane k keeps path[k]
      len = 1;
      while (true) {
        const int want = target[o0 + cur];
        const uint64_t m = __ballot(active && p == cur && tok == want);
        if (m == 0) break;
        const int c = __ffsll((unsigned long long)m) - 1;
        if (lane == len) mine = c;
        ++len;
        cur = c;
      }
      if (lane < len) {
        s_path[lane] = mine;
        path[b * TTV_MAX_NODES + lane] = mine;
        emitted[b * TTV_MAX_NODES + lane] = target[o0 + mine];
      }
      if (lane == 0) path_len[b] = len;
    } else if (lane == 0) {
      *status = TTV_DEV_BAD_PARENT;
    }
    if (lane == 0) s_len = bad ? -1 : len;
  }
  __syncthreads();
  const int len = s_len;
  if (len < 0 || sel == nullptr) {
    if (len >= 0 && sel_len_out && tid == 0) sel_len_out[b] = hist_len[b] + len;
    return;
  }
  const int P = hist_len[b];
  int32_t* row = sel + (size_t)b * sel_stride;
  if (tid < len) row[P + tid] = P + s_path[tid];
  if (tid == 0 && sel_len_out) sel_len_out[b] = P + len;
}

}  // namespace ttv

using namespace ttv;

extern "C" const char* ttv_last_error(void) { return g_error.c_str(); }

extern "C" ttv_status tree_build_mask(const ttv_batch* batch, const int32_t* parent, uint64_t* anc,
                                      int32_t* depth, int32_t* dev_status, void* stream) {
  clear_error();
  ttv_status s = check_batch(batch);
  if (s != TTV_OK) return s;
  if (batch->B == 0 || batch->node_off_h[batch->B] == 0) return TTV_OK;
  TTV_REQUIRE(parent && anc && dev_status, TTV_ERR_INVALID, "tree_build_mask: NULL pointer");
  hipLaunchKernelGGL(mask_kernel, dim3(batch->B), dim3(64), 0, (hipStream_t)stream,
                     batch->node_off_d, parent, anc, depth, dev_status);
  return check_launch("tree_build_mask");
}

extern "C" ttv_status tree_mask_expand_additive(const ttv_batch* batch, int32_t b, const uint64_t* anc,
                                                float masked, float* out, void* stream) {
  clear_error();
  ttv_status s = check_batch(batch);
  if (s != TTV_OK) return s;
  TTV_REQUIRE(b >= 0 && b < batch->B, TTV_ERR_INVALID, "sequence %d outside the batch", b);
  TTV_REQUIRE(anc && out, TTV_ERR_INVALID, "tree_mask_expand_additive: NULL pointer");
  const int o0 = batch->node_off_h[b];
  const int T = batch->node_off_h[b + 1] - o0;
  const int P = batch->hist_len_h[b];
  if (T == 0) return TTV_OK;
  const int W = P + T;
  dim3 grid((W + 255) / 256 < 64 ? (W + 255) / 256 : 64, T);
  hipLaunchKernelGGL(expand_kernel, grid, dim3(256), 0, (hipStream_t)stream, anc + o0, P, T, masked, out);
  return check_launch("tree_mask_expand_additive");
}

extern "C" ttv_status sliding_mask_from_caller(const float* caller, int32_t T, int32_t S, int32_t offset,
                                               int32_t window, float masked, float* out, void* stream) {
  clear_error();
  TTV_REQUIRE(T >= 0 && S >= 0 && offset >= 0, TTV_ERR_INVALID, "sliding_mask_from_caller: T %d, S %d, offset %d", T,
              S, offset);
  TTV_REQUIRE(window >= 1, TTV_ERR_INVALID, "sliding_mask_from_caller: window %d < 1", window);
  TTV_REQUIRE(T <= 65535 && (int64_t)offset + T <= 0x7FFFFFFF, TTV_ERR_INVALID,
              "sliding_mask_from_caller: %d rows at offset %d out of range", T, offset);
  if (T == 0 || S == 0) return TTV_OK;
  TTV_REQUIRE(caller && out, TTV_ERR_INVALID, "sliding_mask_from_caller: NULL pointer");
  const size_t bytes = (size_t)T * S * sizeof(float);
  const uintptr_t a = reinterpret_cast<uintptr_t>(caller), o = reinterpret_cast<uintptr_t>(out);
  TTV_REQUIRE(a == o || a + bytes <= o || o + bytes <= a, TTV_ERR_INVALID,
              "sliding_mask_from_caller: out partly overlaps caller (only out == caller is allowed)");
  dim3 grid((S + 255) / 256 < 64 ? (S + 255) / 256 : 64, T);
  // below the window the band and the caller mask cannot disagree: the caller
  // mask comes back untouched
  if ((int64_t)offset + T <= window) {
    if (a == o) return TTV_OK;
    hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, (hipStream_t)stream, caller, S, out);
  } else {
    hipLaunchKernelGGL(band_kernel, grid, dim3(256), 0, (hipStream_t)stream, caller, S, offset, window, masked, out);
  }
  return check_launch("sliding_mask_from_caller");
}

extern "C" ttv_status tree_accept_walk(const ttv_batch* batch, const int32_t* parent,
                                       const int32_t* token, const int32_t* target_argmax,
                                       int32_t* path, int32_t* path_len, int32_t* emitted,
                                       int32_t* sel, int32_t sel_stride, int32_t* sel_len_out,
                                       int32_t* dev_status, void* stream) {
  clear_error();
  ttv_status s = check_batch(batch);
  if (s != TTV_OK) return s;
  if (batch->B == 0) return TTV_OK;
  TTV_REQUIRE(parent && token && target_argmax && path && path_len && emitted && dev_status,
              TTV_ERR_INVALID, "tree_accept_walk: NULL pointer");
  for (int b = 0; b < batch->B; ++b) {
    const int T = batch->node_off_h[b + 1] - batch->node_off_h[b];
    TTV_REQUIRE(T >= 1, TTV_ERR_INVALID, "tree_accept_walk: sequence %d has an empty tree", b);
    if (sel)
      TTV_REQUIRE(sel_stride >= batch->hist_len_h[b] + T, TTV_ERR_INVALID,
                  "tree_accept_walk: sel_stride %d < P + T = %d for sequence %d", sel_stride,
                  batch->hist_len_h[b] + T, b);
  }
  int max_p = 0;
  for (int b = 0; b < batch->B; ++b) max_p = batch->hist_len_h[b] > max_p ? batch->hist_len_h[b] : max_p;
  const int prefix_chunks = sel ? (max_p + kWalkPrefixChunk - 1) / kWalkPrefixChunk : 0;
  hipLaunchKernelGGL(walk_kernel, dim3(1 + prefix_chunks, batch->B), dim3(256), 0, (hipStream_t)stream,
                     batch->node_off_d,
                     batch->hist_len_d, parent, token, target_argmax, path, path_len, emitted, sel,
                     sel_stride, sel_len_out, dev_status);
  return check_launch("tree_accept_walk");
}

extern "C" ttv_status kv_can_gather(const ttv_kv_layer* layers, int32_t n_layers) {
  clear_error();
  TTV_REQUIRE(layers != nullptr || n_layers == 0, TTV_ERR_INVALID, "kv_can_gather: layers is NULL");
  for (int l = 0; l < n_layers; ++l) {
    const ttv_kv_layer& L = layers[l];
    TTV_REQUIRE(L.dtype == TTV_F32 || L.dtype == TTV_BF16 || L.dtype == TTV_I8, TTV_ERR_UNSUPPORTED,
                "layer %d: unknown KV dtype %d", l, L.dtype);
    TTV_REQUIRE(L.k && L.v, TTV_ERR_UNSUPPORTED, "layer %d: no dense K/V buffer to gather", l);
    TTV_REQUIRE(L.Hkv > 0 && L.D > 0 && L.cap >= 0, TTV_ERR_INVALID, "layer %d: bad shape", l);
    const int esz = L.dtype == TTV_F32 ? 4 : L.dtype == TTV_BF16 ? 2 : 1;
    TTV_REQUIRE((L.D * esz) % 16 == 0, TTV_ERR_UNSUPPORTED,
                "layer %d: a %d-byte row is not a whole number of 16-byte chunks", l, L.D * esz);
    TTV_REQUIRE(L.D * esz <= kMaxGatherRowBytes, TTV_ERR_UNSUPPORTED,
                "layer %d: %d-byte rows are wider than the gather moves (at most %d bytes)", l, L.D * esz,
                kMaxGatherRowBytes);
    if (L.dtype == TTV_I8)
      TTV_REQUIRE(L.k_scale && L.v_scale, TTV_ERR_UNSUPPORTED,
                  "layer %d: int8 cache without per-token scale sidecars; moving codes without "
                  "their scales would decode survivors against another token's scale",
                  l);
  }
  return TTV_OK;
}
