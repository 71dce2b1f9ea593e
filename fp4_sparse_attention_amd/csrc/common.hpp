// Shared device helpers and host-side argument checks for libcsa2 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

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

// 16-byte streaming (non-temporal) load
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr int kLatent = 512;        // latent KV channels
constexpr int kCodesRow = 256;      // packed FP4 bytes per latent row
constexpr int kScalesRow = 32;      // E4M3 scale bytes per latent row
constexpr int kIndexDim = 64;       // indexer key / query bytes
constexpr int kWindowMax = 128;     // sliding-window bound

// ----------------------------------------------------------------------------
// scalar conversions
// ----------------------------------------------------------------------------
// E4M3FN byte -> fp32, exact.  Normal codes: exponent e (bias 7) and mantissa m
// map to fp32 exponent e+120; subnormal codes are m * 2^-9; 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t mag = b & 0x7Fu;
  float normal = __uint_as_float((mag << 20) + (120u << 23));
  float sub = (float)mag * 0.001953125f;
  float v = mag >= 8u ? normal : sub;
  v = mag == 0x7Fu ? __builtin_nanf("") : v;
  return (b & 0x80u) ? -v : v;
}

// ----------------------------------------------------------------------------
// wave-level helpers (wave64)
// ----------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// lane l's value and lane (l ^ 16)'s, resp. (l ^ 32)'s, in one VALU step each
// (gfx950's v_permlane16_swap / v_permlane32_swap on two copies of v: every
// lane ends with the pair, in an order that depends on the lane), so a
// reduction over those lanes needs no LDS round trip; a + b and max(a, b)
// give both lanes of a pair the same bits
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v from the lane selected by a DPP control (0 where the source lane is
// outside the row or the destination row is masked off)
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, true);
}

// inclusive prefix sum over the 64 lanes of a wave: shifts within each row of
// 16 lanes, then the row totals broadcast forward (row_bcast:15, row_bcast:31)
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_u32<0x111>(x);          // row_shr:1
  x += dpp_u32<0x112>(x);          // row_shr:2
  x += dpp_u32<0x114>(x);          // row_shr:4
  x += dpp_u32<0x118>(x);          // row_shr:8
  x += dpp_u32<0x142, 0xA>(x);     // row_bcast:15 -> rows 1, 3
  x += dpp_u32<0x143, 0xC>(x);     // row_bcast:31 -> rows 2, 3
  return x;
}

// a value that is the same in every lane, moved to a scalar register so that
// tests on it compile to scalar compares and branches
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(x), 63);
}

// number of set bits of a wave-wide mask in the lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// block-wide exclusive prefix sum, 1024 threads (16 waves); wt holds >= 16 words
__device__ __forceinline__ uint32_t block_scan_1024(uint32_t v, uint32_t* wt, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t t = wt[w];
    base += w < wave ? t : 0u;
    tot += t;
  }
  total = tot;
  __syncthreads();
  return base + inc - v;
}

// block-wide exclusive prefix sum, 256 threads (4 waves); wt holds >= 4 words
__device__ __forceinline__ uint32_t block_scan_256(uint32_t v, uint32_t* wt, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  const uint32_t t0 = wt[0], t1 = wt[1], t2 = wt[2], t3 = wt[3];
  total = t0 + t1 + t2 + t3;
  const uint32_t base = (wave > 0 ? t0 : 0u) + (wave > 1 ? t1 : 0u) + (wave > 2 ? t2 : 0u);
  __syncthreads();
  return base + inc - v;
}

// the same digit search by 256 threads (kNB / 256 bins per thread)
template <int kNB>
__device__ __forceinline__ void find_bin_256(const uint32_t* hh, uint32_t need, uint32_t* wt, uint32_t* out2) {
  constexpr int kPer = kNB / 256;
  uint32_t c[kPer], local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = hh[kNB - 1 - kPer * threadIdx.x - j];
    local += c[j];
  }
  uint32_t total;
  const uint32_t excl = block_scan_256(local, wt, total);
  if (excl < need && need <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (acc < need && need <= acc + c[j]) {
        out2[0] = (uint32_t)(kNB - 1 - kPer * threadIdx.x - j);
        out2[1] = acc;
      }
      acc += c[j];
    }
  }
}

// digit search over a histogram in LDS by 1024 threads: bins are walked from the
// top, thread t owns bins nb-1-(nb/1024)t-j; returns the bin holding the need-th
// largest entry and the count above it (need >= 1 and <= the histogram total)
template <int kNB>
__device__ __forceinline__ void find_bin_1024(const uint32_t* hh, uint32_t need, uint32_t* wt, uint32_t* out2) {
  constexpr int kPer = kNB / 1024;
  uint32_t c[kPer], local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = hh[kNB - 1 - kPer * threadIdx.x - j];
    local += c[j];
  }
  uint32_t total;
  const uint32_t excl = block_scan_1024(local, wt, total);
  if (excl < need && need <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (acc < need && need <= acc + c[j]) {
        out2[0] = (uint32_t)(kNB - 1 - kPer * threadIdx.x - j);
        out2[1] = acc;
      }
      acc += c[j];
    }
  }
}

// ----------------------------------------------------------------------------
// order-preserving 32-bit keys of fp32 scores (Top-K selection): positive
// scores get the sign bit set, negative ones are bit-inverted, -0 ranks as +0;
// -inf and NaN map to key 0, which no visible score reaches (the smallest,
// -FLT_MAX, maps to 0x00800000)
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = x == 0.0f ? 0u : __float_as_uint(x);     // -0 ranks equal to +0
  if (x != x || x == -__builtin_inff()) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// inverse of score_key for visible keys (a -0 score comes back as +0)
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// ----------------------------------------------------------------------------
// paged caches: sequence b's logical position p lives in physical row
// table[b][p / page] * page + p % page of a page pool (table == null: the dense
// layout, row b T + p).  Unmapped blocks (negative entries) hold no positions.
// ----------------------------------------------------------------------------
struct PageMap {
  const int32_t* table;   // [B][max_blocks] or null
  int64_t max_blocks;
  int32_t page;           // positions per page, a multiple of 128
};

__device__ __forceinline__ int64_t phys_row(const PageMap& pm, int seq, int64_t T, int64_t p) {
  if (!pm.table) return (int64_t)seq * T + p;
  const int64_t blk = p / pm.page;
  if (blk >= pm.max_blocks) return -1;
  const int32_t pg = pm.table[(int64_t)seq * pm.max_blocks + blk];
  return pg < 0 ? -1 : (int64_t)pg * pm.page + (p - blk * pm.page);
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

// Compute units of the current device, queried once per device (each GPU the
// library runs on keeps its own entry); 256, the MI355X count, if the query fails.
constexpr int kMaxDevices = 64;
inline int device_cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev >= 0) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace csa2
