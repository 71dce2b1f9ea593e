// FP4 KV-cache pack / unpack kernels (E2M1 elements, one E4M3 scale per 16
// channels, no global scale -- the NVFP4-style layout of the KV-cache paragraph
// of the MarkTechPost retelling of DeepSeek-V4.1-Flash).
//
// Work split: the pack gives a thread 32 consecutive channels (two scale
// blocks); the unpack gives a lane 8 channels, so that every wave store writes
// a contiguous 1 KB of bf16 (with 32 channels per lane each store instruction
// covered a 64-byte-strided quarter of 4 KB, and with nontemporal stores the
// unpack ran at 1.4 TB/s).  The kernels are HBM-bound: the pack rounds with
// gfx950's FP4 conversion instruction (about five lane-ops per element, see
// pack_block), the unpack with integer bit work.
#include "common.hpp"

namespace csa2 {

// Nearest E4M3FN code to a non-negative fp32 value, ties to the even code,
// finite values >= 448 saturate to 0x7E.  The input is the correctly rounded
// fp32 quotient amax/6 with amax a bf16 value: a tie of the E4M3 grid has at
// most 5 significant bits, so the quotient is either exactly a tie (and exact
// in fp32) or far (>= 2^-16 relative) from one, and rounding the fp32 value
// decides as the exact quotient would.
__device__ __forceinline__ uint32_t e4m3_code_nonneg(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0.015625f) {                       // below 2^-6: subnormal grid m * 2^-9
    return (uint32_t)rintf(v * 512.0f);      // 0..8 (8 is 2^-6 = code 0x08)
  }
  uint32_t bits = __float_as_uint(v);
  uint32_t e = (bits >> 23) - 120u;          // E4M3 exponent field, 1..15
  uint32_t m = bits & 0x7FFFFFu;
  uint32_t code = (e << 3) | (m >> 20);
  uint32_t rem = m & 0xFFFFFu;
  code += (rem > 0x80000u) || (rem == 0x80000u && (code & 1u));
  return code > 0x7Eu ? 0x7Eu : code;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// E2M1 code of x / s, nearest with ties to even, saturating at 6, from y =
// x * r with r = v_rcp_f32(s) (within 1 ulp of 1/s):
//   * y is within 2^-22 of x / s (relative).  A midpoint m of the E2M1 grid
//     (0.25, 0.75, ..., 5) has at most 3 significant bits, so m s has at most 7
//     and x (bf16, 8 bits) either equals m s or differs from it by at least
//     2^-8 relative;
//   * rounding y to 10 significant bits therefore returns exactly m when x / s
//     is the midpoint m, and keeps every other value on its side of every
//     midpoint (it moves y by at most 2^-10 relative);
//   * v_cvt_scalef32_pk_fp4_f32 with unit scale then rounds to nearest even on
//     the E2M1 grid, saturates magnitudes above 6 (infinities included) to 6,
//     and keeps the sign of zero.
// So the code equals the nearest-even E2M1 value of the exact quotient.
__device__ __forceinline__ float snap10(float y) {
  return __uint_as_float((__float_as_uint(y) + 0x2000u) & 0xFFFFC000u);
}

// one 16-channel block: 8 dwords of packed bf16 pairs -> 2 dwords of nibbles + scale byte
__device__ __forceinline__ void pack_block(const uint32_t* w, uint32_t& lo, uint32_t& hi, uint32_t& sc) {
  // |bf16| orders like its bit pattern: the largest magnitude from packed 16-bit maxima
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  const uint32_t amax_bits = max((uint32_t)m2[0], (uint32_t)m2[1]);
  const float amax = __uint_as_float(amax_bits << 16);
  // a NaN anywhere in the block (|bits| above the infinity pattern) gives the
  // NaN scale 0x7F and every magnitude code 0 (the whole block decodes to NaN);
  // infinities saturate like large finite values
  const uint32_t code = amax_bits > 0x7F80u ? 0x7Fu : e4m3_code_nonneg(__fdiv_rn(amax, 6.0f));
  uint32_t out[2] = {0u, 0u};
  if (code == 0x7Fu) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t n0 = (w[i] >> 12) & 8u, n1 = (w[i] >> 28) & 8u;
      out[i >> 2] |= (n0 | (n1 << 4)) << (8 * (i & 3));
    }
  } else {
    // a zero scale (amax / 6 below half the smallest E4M3 step) takes every magnitude to 0
    const float s = e4m3_to_f32(code);
    const float r = code == 0u ? 0.0f : __builtin_amdgcn_rcpf(s);
    // channels 2i (low nibble) and 2i + 1 of pair i into byte i % 4 of out[i / 4]
    auto lo_f = [&](int i) { return snap10(__uint_as_float(w[i] << 16) * r); };
    auto hi_f = [&](int i) { return snap10(__uint_as_float(w[i] & 0xFFFF0000u) * r); };
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t d = 0u;
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, lo_f(4 * q + 0), hi_f(4 * q + 0), 1.0f, 0);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, lo_f(4 * q + 1), hi_f(4 * q + 1), 1.0f, 1);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, lo_f(4 * q + 2), hi_f(4 * q + 2), 1.0f, 2);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, lo_f(4 * q + 3), hi_f(4 * q + 3), 1.0f, 3);
      out[q] = d;
    }
  }
  lo = out[0];
  hi = out[1];
  sc = code;
}

// Pack: one thread owns NB scale blocks (16 NB consecutive channels) of one
// row: 32 NB bytes of bf16 in (plain loads: nontemporal ones were 8% slower),
// 8 NB bytes of codes and NB scale bytes out.  (8 channels per lane, with fully
// contiguous wave accesses and the block amax shared across a lane pair, ran
// slower with threshold-compare rounding: the per-block scale work then
// repeats every 8 channels.)
template <int NB>
__global__ void __launch_bounds__(256)
fp4_pack_kernel(const uint16_t* __restrict__ x, int64_t n_rows, int parts_per_row, int64_t x_stride,
                uint8_t* __restrict__ codes, int64_t codes_stride, uint8_t* __restrict__ scales,
                int64_t scales_stride, const int64_t* __restrict__ out_rows) {
  // (row, part) of this thread's index, advanced by the grid stride without a division per step
  const int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int64_t step_rows = step / parts_per_row;
  const int step_p = (int)(step - step_rows * parts_per_row);
  int64_t row = g0 / parts_per_row;
  int part = (int)(g0 - row * parts_per_row);
  for (; row < n_rows; row += step_rows, part += step_p) {
    if (part >= parts_per_row) {
      part -= parts_per_row;
      ++row;
      if (row >= n_rows) break;
    }
    // output row: the input row's own, or (scatter) out_rows[row]; a negative entry skips the row
    const int64_t orow = out_rows ? out_rows[row] : row;
    if (orow < 0) continue;
    const uint4* src = reinterpret_cast<const uint4*>(x + row * x_stride + part * 16 * NB);
    uint4 v[2 * NB];
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) v[i] = src[i];
    uint32_t c[2 * NB], sc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint32_t w[8] = {v[2 * b].x, v[2 * b].y, v[2 * b].z, v[2 * b].w,
                             v[2 * b + 1].x, v[2 * b + 1].y, v[2 * b + 1].z, v[2 * b + 1].w};
      pack_block(w, c[2 * b], c[2 * b + 1], sc[b]);
    }
    if constexpr (NB == 2) {
      *reinterpret_cast<uint4*>(codes + orow * codes_stride + part * 16) = make_uint4(c[0], c[1], c[2], c[3]);
      *reinterpret_cast<uint16_t*>(scales + orow * scales_stride + part * 2) = (uint16_t)(sc[0] | (sc[1] << 8));
    } else {
      *reinterpret_cast<uint2*>(codes + orow * codes_stride + part * 8) = make_uint2(c[0], c[1]);
      scales[orow * scales_stride + part] = (uint8_t)sc[0];
    }
  }
}

// Two E2M1 nibbles of a byte -> two fp32 values, exact.  Bit form of an E2M1
// magnitude m: m = 0 -> 0, m = 1 -> 0.5, m >= 2 -> exponent (m >> 1) - 1 and
// mantissa bit (m & 1), i.e. fp32 bits (m + 252) << 22.
__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  uint32_t mag = nib & 7u;
  uint32_t b = (mag + 252u) << 22;
  b = mag >= 2u ? b : (mag ? 0x3F000000u : 0u);
  return __uint_as_float(b | ((nib & 8u) << 28));
}

// Unpack: lane g owns 8 channels of one row (4 code bytes + the block's scale
// byte in, 16 bytes of bf16 out), so every wave store writes 1 KB contiguously.
__global__ void __launch_bounds__(256)
fp4_unpack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t n_rows,
                  int chunks_per_row, int C, uint16_t* __restrict__ x) {
  const int64_t g0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  const int64_t step_rows = step / chunks_per_row;
  const int step_c = (int)(step - step_rows * chunks_per_row);
  int64_t row = g0 / chunks_per_row;
  int c = (int)(g0 - row * chunks_per_row);
  for (; row < n_rows; row += step_rows, c += step_c) {
    if (c >= chunks_per_row) {
      c -= chunks_per_row;
      ++row;
      if (row >= n_rows) break;
    }
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + row * (C / 2) + 4 * c);
    const float s = e4m3_to_f32(scales[row * (C / 16) + (c >> 1)]);
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (cw >> (8 * j)) & 0xFFu;
      const float a = e2m1_to_f32(byte & 0xFu) * s;      // exact: <= 6 significant bits
      const float b = e2m1_to_f32(byte >> 4) * s;
      out[j] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
    }
    *reinterpret_cast<uint4*>(x + row * C + 8 * c) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// Decode-time append, one workgroup per sequence: the new token's latent row
// packed into its cache row (16 threads x 32 channels), its indexer key copied
// (4 x 16 bytes), and for each layer its window row written to both slots of a
// mirrored ring of 2 W rows (slots t mod W and t mod W + W), so that the last
// min(W, t + 1) rows always sit contiguously at [start, start + len) with
// start = (t + 1) mod W once t >= W - 1 (0 before) -- the contiguous window the
// attention calls read.  The window bounds of every layer are updated too.
__global__ void __launch_bounds__(256)
decode_append_kernel(int B, int L, const uint16_t* __restrict__ new_latent, const int64_t* __restrict__ cache_rows,
                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const uint8_t* __restrict__ new_keys,
                     uint8_t* __restrict__ k_idx, const uint16_t* __restrict__ new_window, uint16_t* __restrict__ swa,
                     int S, const int64_t* __restrict__ tok_pos, int32_t* __restrict__ swa_start,
                     int32_t* __restrict__ swa_len) {
  constexpr int W = kWindowMax;
  const int b = blockIdx.x, tid = threadIdx.x;
  // every load issued first, at addresses valid for every thread (the branches come after): the row and the
  // token position, this thread's part of the latent row (pack threads) or of the key, and its first window
  // element; behind branches they had made the compiler wait for each in turn
  const int64_t row = cache_rows[b];
  const int64_t t = new_window ? tok_pos[b] : -1;
  const uint4* src = reinterpret_cast<const uint4*>(new_latent + (int64_t)b * kLatent + (tid & 15) * 32);
  const uint4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
  const uint4 kv = new_keys ? *reinterpret_cast<const uint4*>(new_keys + (int64_t)b * kIndexDim + 16 * (tid & 3))
                            : make_uint4(0u, 0u, 0u, 0u);
  const int e0 = tid < L * 64 ? tid : 0;
  const uint4 wv0 = new_window ? reinterpret_cast<const uint4*>(new_window + ((int64_t)(e0 >> 6) * B + b) * kLatent)[e0 & 63]
                               : make_uint4(0u, 0u, 0u, 0u);
  if (row >= 0 && tid < 16) {
    const uint32_t w0[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const uint32_t w1[8] = {v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
    uint32_t c0, c1, c2, c3, s0, s1;
    pack_block(w0, c0, c1, s0);
    pack_block(w1, c2, c3, s1);
    *reinterpret_cast<uint4*>(codes + row * kCodesRow + tid * 16) = make_uint4(c0, c1, c2, c3);
    *reinterpret_cast<uint16_t*>(scales + row * kScalesRow + tid * 2) = (uint16_t)(s0 | (s1 << 8));
  } else if (row >= 0 && tid < 20 && new_keys) {
    const int q = tid - 16;
    *reinterpret_cast<uint4*>(k_idx + row * kIndexDim + 16 * q) = kv;
  }
  if (!new_window) return;
  if (t < 0) return;
  const int slot = (int)(t % W);
  for (int e = tid; e < L * 64; e += 256) {
    const int l = e >> 6, c = e & 63;
    const int64_t lb = (int64_t)l * B + b;
    const uint4 v = e == tid ? wv0 : reinterpret_cast<const uint4*>(new_window + lb * kLatent)[c];
    uint16_t* ring = swa + lb * S * kLatent;
    reinterpret_cast<uint4*>(ring + (int64_t)slot * kLatent)[c] = v;
    reinterpret_cast<uint4*>(ring + (int64_t)(slot + W) * kLatent)[c] = v;
  }
  for (int l = tid; l < L; l += 256) {
    swa_start[(int64_t)l * B + b] = t >= W - 1 ? (int32_t)((t + 1) % W) : 0;
    swa_len[(int64_t)l * B + b] = (int32_t)(t + 1 < W ? t + 1 : W);
  }
}

// Two scale blocks per pack thread (one block per thread measured 317 vs 306 us
// at 2^20 rows).  The grids give every item its own thread up to 256
// workgroups per compute unit (2^20 rows: 65,536 workgroups); a grid-stride
// loop with 16 workgroups per CU ran the pack at 306 us, 32 at 295, 128 at 288,
// one item per thread at 280.
constexpr int kPackNB = 2;
constexpr int64_t kStreamWgPerCu = 256;

static int stream_grid(int64_t total_threads) {
  int64_t blocks = (total_threads + 255) / 256;
  const int64_t cap = 256 * kStreamWgPerCu;   // workgroups, grid-stride beyond
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace csa2

using namespace csa2;

extern "C" csa2_status csa2_fp4_pack(const uint16_t* x, int64_t n_rows, int32_t C, int64_t x_row_stride,
                                     uint8_t* codes, int64_t codes_row_stride, uint8_t* scales,
                                     int64_t scales_row_stride, void* stream) {
  if (n_rows < 0) return CSA2_EINVAL;
  if (C <= 0 || C % 32 != 0) return CSA2_ESHAPE;
  if (x_row_stride < C || x_row_stride % 8 != 0) return CSA2_EINVAL;
  if (codes_row_stride < C / 2 || codes_row_stride % 16 != 0) return CSA2_EINVAL;
  if (scales_row_stride < C / 16 || scales_row_stride % 2 != 0) return CSA2_EINVAL;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return CSA2_EALIGN;
  const int parts = C / (16 * kPackNB);
  fp4_pack_kernel<kPackNB><<<stream_grid(n_rows * parts), 256, 0, (hipStream_t)stream>>>(
      x, n_rows, parts, x_row_stride, codes, codes_row_stride, scales, scales_row_stride, nullptr);
  return launch_status();
}

extern "C" csa2_status csa2_fp4_pack_rows(const uint16_t* x, int64_t n_rows, int32_t C, int64_t x_row_stride,
                                          const int64_t* out_rows, uint8_t* codes, int64_t codes_row_stride,
                                          uint8_t* scales, int64_t scales_row_stride, void* stream) {
  if (n_rows < 0) return CSA2_EINVAL;
  if (C <= 0 || C % 32 != 0) return CSA2_ESHAPE;
  if (x_row_stride < C || x_row_stride % 8 != 0) return CSA2_EINVAL;
  if (codes_row_stride < C / 2 || codes_row_stride % 16 != 0) return CSA2_EINVAL;
  if (scales_row_stride < C / 16 || scales_row_stride % 2 != 0) return CSA2_EINVAL;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !out_rows || !codes || !scales) return CSA2_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(out_rows, 8)) return CSA2_EALIGN;
  const int parts = C / (16 * kPackNB);
  fp4_pack_kernel<kPackNB><<<stream_grid(n_rows * parts), 256, 0, (hipStream_t)stream>>>(
      x, n_rows, parts, x_row_stride, codes, codes_row_stride, scales, scales_row_stride, out_rows);
  return launch_status();
}

extern "C" csa2_status csa2_fp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, int32_t C,
                                       uint16_t* x, void* stream) {
  if (n_rows < 0) return CSA2_EINVAL;
  if (C <= 0 || C % 32 != 0) return CSA2_ESHAPE;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return CSA2_EALIGN;
  const int chunks = C / 8;
  fp4_unpack_kernel<<<stream_grid(n_rows * chunks), 256, 0, (hipStream_t)stream>>>(
      codes, scales, n_rows, chunks, C, x);
  return launch_status();
}

extern "C" csa2_status csa2_decode_append(int32_t B, int32_t L, const uint16_t* new_latent, const int64_t* cache_rows,
                                          uint8_t* codes, uint8_t* scales, const uint8_t* new_keys, uint8_t* k_idx,
                                          const uint16_t* new_window, uint16_t* swa, int32_t S,
                                          const int64_t* tok_pos, int32_t* swa_start, int32_t* swa_len,
                                          void* stream) {
  if (B < 0 || L < 0) return CSA2_EINVAL;
  if (B == 0) return CSA2_OK;
  if (!new_latent || !cache_rows || !codes || !scales) return CSA2_EINVAL;
  if (new_keys && !k_idx) return CSA2_EINVAL;
  if (new_window) {
    if (L == 0 || !swa || !tok_pos || !swa_start || !swa_len) return CSA2_EINVAL;
    if (S < 2 * kWindowMax) return CSA2_ESHAPE;
  }
  if (!aligned(new_latent, 16) || !aligned(cache_rows, 8) || !aligned(codes, 16) || !aligned(scales, 2) ||
      (new_keys && (!aligned(new_keys, 16) || !aligned(k_idx, 16))) ||
      (new_window && (!aligned(new_window, 16) || !aligned(swa, 16) || !aligned(tok_pos, 8) ||
                      !aligned(swa_start, 4) || !aligned(swa_len, 4))))
    return CSA2_EALIGN;
  decode_append_kernel<<<B, 256, 0, (hipStream_t)stream>>>(B, L, new_latent, cache_rows, codes, scales, new_keys,
                                                            k_idx, new_window, swa, S, tok_pos, swa_start, swa_len);
  return launch_status();
}
