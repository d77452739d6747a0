// Shared host/device helpers for libttv (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/ttv.h"

namespace ttv {

// ---------------------------------------------------------------- errors ----
void set_error(const char* fmt, ...);
void clear_error();

inline ttv_status fail(ttv_status s, const char* msg) {
  set_error("%s", msg);
  return s;
}

#define TTV_REQUIRE(cond, code, ...)  \
  do {                                \
    if (!(cond)) {                    \
      ::ttv::set_error(__VA_ARGS__);  \
      return code;                    \
    }                                 \
  } while (0)

inline ttv_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return TTV_ERR_HIP;
  }
  return TTV_OK;
}

// Validates the host-side description of a batch of trees.
ttv_status check_batch(const ttv_batch* batch, bool need_device = true);

// ------------------------------------------------------------ constants ----
constexpr int kWave = 64;
// Widest K (or V) row the gather moves: one 256-thread pass of 16-byte pieces
// (the out-of-place take copies a row per pass; the in-place form holds at
// least one whole row per chunk).
constexpr int kMaxGatherRowBytes = 4096;
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, round-robin workgroup dispatch

// Remap a linear workgroup id so that consecutive logical slots land on the
// same XCD: the hardware deals workgroups to XCDs round-robin (wg % 8), so
// logical slot = (wg % 8) * ceil(n/8) + wg / 8 gives each XCD one contiguous
// block of slots (and hence one L2 for neighbouring work). Slots >= n are
// returned as -1.
__device__ __forceinline__ int xcd_slot(int wg, int n) {
  const int per = (n + kNumXcd - 1) / kNumXcd;
  const int x = wg % kNumXcd;
  const int j = wg / kNumXcd;
  // the grid is padded to a multiple of 8; XCD x gets slots [x*per, x*per+per)
  const int s = x * per + j;
  return (j < per && s < n) ? s : -1;
}

// -------------------------------------------------------------- numbers ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float fp16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __asm__ volatile("" ::: "memory");
}

// Direct global -> LDS loads of 16 bytes per lane; lane i lands at lds + 16 i
// (lds must be wave-uniform). Issued as inline asm on purpose: the compiler
// treats its own LDS-DMA builtin as possibly aliasing every later LDS read and
// would wait for all outstanding DMAs (vmcnt 0) before each tile, which
// serialises the ring. Completion is tracked explicitly with wait_vmcnt; the
// memory clobber keeps every other memory access in program order.
__device__ __forceinline__ uint32_t lds_u32(const void* lds) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(lds))));
}
// scalar base (wave-uniform) + 32-bit per-lane byte offset; lds: LDS byte
// address (wave-uniform)
__device__ __forceinline__ void dma16_at(const void* sbase, uint32_t voff, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                   : "memory");
}
// per-lane 64-bit address
__device__ __forceinline__ void dma16v_at(const void* g, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
}  // namespace ttv
