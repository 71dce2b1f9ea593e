// Shared device helpers and host-side argument checks for libcsa2 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "csa2.h"

namespace csa2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming (non-temporal) load / store
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

constexpr int kLatent = 512;        // latent KV channels
constexpr int kCodesRow = 256;      // packed FP4 bytes per latent row
constexpr int kScalesRow = 32;      // E4M3 scale bytes per latent row
constexpr int kIndexDim = 64;       // indexer key / query bytes
constexpr int kWindowMax = 128;     // sliding-window bound

// ----------------------------------------------------------------------------
// scalar conversions
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// E4M3FN byte (non-NaN) -> fp32, exact.  Normal codes: exponent e (bias 7) and
// mantissa m map to fp32 exponent e+120; subnormal codes are m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t mag = b & 0x7Fu;
  float normal = __uint_as_float((mag << 20) + (120u << 23));
  float sub = (float)mag * 0.001953125f;
  float v = mag >= 8u ? normal : sub;
  return (b & 0x80u) ? -v : v;
}

// ----------------------------------------------------------------------------
// wave-level helpers (wave64)
// ----------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// ----------------------------------------------------------------------------
// host-side checks
// ----------------------------------------------------------------------------
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline csa2_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? CSA2_OK : CSA2_ELAUNCH;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace csa2
