// Indexer tile arithmetic shared by every scoring kernel, so that all of them
// round identically: 32 keys per tile on v_mfma_f32_16x16x32_f16, E4M3 widened
// to f16 exactly.
//
// Layout.  Lane l = 16 g + n (g = l / 16, n = l % 16) holds bytes
// [16 g, 16 g + 16) of the tile's keys n and n + 16: a wave reads the tile's
// 2 KB as two 1 KB loads that each cover 16 whole keys.  Each half of the tile
// (keys 0-15, keys 16-31) takes two k-steps; in k-step s the lane supplies its
// bytes 8 s .. 8 s + 7 as k = 8 g .. 8 g + 7 (the query operand uses the same
// map in row 0 of A, rows 1-15 zero).  So a score sums channels
// {16 g + 8 s + j : g < 4, j < 8} in step s and adds the two steps in fp32.
// Output: C[m][n] sits in register m % 4 of lane 16 (m / 4) + n, so the tile's
// scores are register 0 of lanes 0-15 (key n in the first accumulator, key
// n + 16 in the second).
#pragma once

#include "common.hpp"

namespace csa2 {

constexpr int kTile = 32;          // keys per tile
constexpr int kUnroll = 4;         // tiles in flight per wave

// 16 E4M3 bytes -> two f16x8 operands (bytes 0-7, bytes 8-15), exact
__device__ __forceinline__ void fp8x16_to_f16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, f16x8* out) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w2, 1.0f, false);
  const f16x2 f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w2, 1.0f, true);
  const f16x2 g = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w3, 1.0f, false);
  const f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w3, 1.0f, true);
  out[0] = f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  out[1] = f16x8{e[0], e[1], f[0], f[1], g[0], g[1], h[0], h[1]};
}

// the lane's 16 bytes of one key (p already offset by 16 g): nontemporal loads
// by default (measured best for the candidate scan and the gathers), plain
// loads with kNT = false (best for the scores-only scan)
template <bool kNT = true>
__device__ __forceinline__ uint4 load_key_part(const uint8_t* p) {
  return kNT ? ld_nt16(p) : *reinterpret_cast<const uint4*>(p);
}

// a tile's B data in one register set: part of key n, then part of key n + 16
__device__ __forceinline__ i32x8 tile_pair(uint4 lo, uint4 hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// scores of keys n and n + 16 (valid in lanes 0-15)
__device__ __forceinline__ float2 mfma_score(const f16x8* a, const i32x8& kb) {
  f16x8 lo[2], hi[2];
  fp8x16_to_f16((uint32_t)kb[0], (uint32_t)kb[1], (uint32_t)kb[2], (uint32_t)kb[3], lo);
  fp8x16_to_f16((uint32_t)kb[4], (uint32_t)kb[5], (uint32_t)kb[6], (uint32_t)kb[7], hi);
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
  c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], lo[0], c0, 0, 0, 0);
  c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], lo[1], c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], hi[0], c1, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], hi[1], c1, 0, 0, 0);
  return make_float2(c0[0], c1[0]);
}

// the A operands of one query row: lanes 0, 16, 32, 48 hold its bytes 16 g ..
// 16 g + 15, every other lane zero
__device__ __forceinline__ void query_operands(const uint8_t* q_row, int lane, f16x8* a) {
  uint4 x = make_uint4(0, 0, 0, 0);
  if ((lane & 15) == 0) x = *reinterpret_cast<const uint4*>(q_row + 16 * (lane >> 4));
  fp8x16_to_f16(x.x, x.y, x.z, x.w, a);
}

// The FP8 matrix instruction on the same layout, for csa2_index_full_fp8 only:
// the raw E4M3 bytes go in as operands, with no widening.  This is not the
// arithmetic above -- the instruction does not form the exact sum of its 32
// products (on unit-normal E4M3 data about half the scores differ from the
// exactly rounded value, by up to about 2^-15 sum |q k|) -- so no selection in
// this library uses it.
__device__ __forceinline__ void query_operands_fp8(const uint8_t* q_row, int lane, long* a8) {
  uint4 x = make_uint4(0, 0, 0, 0);
  if ((lane & 15) == 0) x = *reinterpret_cast<const uint4*>(q_row + 16 * (lane >> 4));
  a8[0] = (long)(((uint64_t)x.y << 32) | x.x);
  a8[1] = (long)(((uint64_t)x.w << 32) | x.z);
}

__device__ __forceinline__ float2 mfma_score_fp8(const long* a8, const i32x8& kb) {
  auto pair = [](int lo, int hi) { return (long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo); };
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
  c0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8[0], pair(kb[0], kb[1]), c0, 0, 0, 0);
  c0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8[1], pair(kb[2], kb[3]), c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8[0], pair(kb[4], kb[5]), c1, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8[1], pair(kb[6], kb[7]), c1, 0, 0, 0);
  return make_float2(c0[0], c1[0]);
}

}  // namespace csa2
