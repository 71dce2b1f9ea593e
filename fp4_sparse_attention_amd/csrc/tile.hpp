// Indexer tile arithmetic shared by the scoring kernels: 32 keys per
// v_mfma_f32_32x32x16_f16 tile, E4M3 widened to f16 exactly, the query in one
// column of A.  Lane l owns key column l % 32 and one 32-byte half of the
// 64-byte key; the score of key column c sits in register 0 of lane c.
#pragma once

#include "common.hpp"

namespace csa2 {

constexpr int kTile = 32;          // keys per MFMA tile
constexpr int kUnroll = 4;         // tiles in flight per wave

// 32 E4M3 bytes (8 dwords) -> four f16x8 MFMA operands, exact
__device__ __forceinline__ void fp8x32_to_f16(const i32x8& v, f16x8* out) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t w0 = (uint32_t)v[2 * ks], w1 = (uint32_t)v[2 * ks + 1];
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    out[ks] = f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

// score tile: sum over the four 16-element k-steps of the lane's 32-byte half
__device__ __forceinline__ f32x16 mfma_score(const f16x8* a, const i32x8& kb) {
  f16x8 b[4];
  fp8x32_to_f16(kb, b);
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks], b[ks], acc, 0, 0, 0);
  return acc;
}

// the lane's 32 bytes of a key: nontemporal loads by default (measured best for
// the candidate scan and the gathers), plain loads with kNT = false (best for
// the scores-only scan, 108 vs 115 us at 8 x 1M)
template <bool kNT = true>
__device__ __forceinline__ i32x8 load_half_key(const uint8_t* p) {
  uint4 x = kNT ? ld_nt16(p) : *reinterpret_cast<const uint4*>(p);
  uint4 y = kNT ? ld_nt16(p + 16) : *reinterpret_cast<const uint4*>(p + 16);
  i32x8 r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}

// the query row's four A operands (its 64 bytes in column 0, zero elsewhere)
__device__ __forceinline__ void query_operands(const uint8_t* q_row, int lane, f16x8* a) {
  i32x8 araw = {0, 0, 0, 0, 0, 0, 0, 0};
  if ((lane & 31) == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(q_row + 32 * (lane >> 5));
    const uint4 x = q[0], y = q[1];
    araw[0] = x.x; araw[1] = x.y; araw[2] = x.z; araw[3] = x.w;
    araw[4] = y.x; araw[5] = y.y; araw[6] = y.z; araw[7] = y.w;
  }
  fp8x32_to_f16(araw, a);
}

}  // namespace csa2
