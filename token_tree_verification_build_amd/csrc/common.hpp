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

}  // namespace ttv
