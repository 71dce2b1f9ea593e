// Query absorption and output unabsorption for absorbed multi-head latent
// attention: every head attends over the one 512-channel latent row per
// position (the shared main KV of the HN summary's key points; the
// MarkTechPost retelling, paragraph 3), with 128-d head queries and outputs.
// Head h's key of a latent row x is W_UK,h x and its value W_UV,h x
// (W [128][512] per head), so
//   absorb:    q_lat[r][h][c] = sum_d q[r][h][d] W_UK[h][d][c]     (128 -> 512)
//   unabsorb:  o[r][h][d]     = sum_c W_UV[h][d][c] o_lat[r][h][c] (512 -> 128)
//
// Both are per-head matrix products on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  bf16 inputs times bf16 weights are exact products.  At decode
// sizes (a few rows per head) the weights dominate the bytes, so each head's
// weight matrix is split over four workgroups (H x 4 workgroups fill the chip
// at H = 64), and each weight byte is read once per 64 rows.
//   * absorb: C^T[c][r] = W_UK^T[c][d] q^T[d][r].  Workgroup (h, s) stages
//     W_UK[h][0..128)[128 s .. 128 s + 128) (32 KB) in LDS; wave w owns channels
//     128 s + 32 w + [0, 32).  The A operand needs 8 consecutive d of one channel
//     per lane, a column of W_UK[h], read with ds_read_b64_tr_b16 (gfx950's
//     transposing LDS read).  The fp32 result is rounded once to bf16 (round to
//     nearest even).
//   * unabsorb: C^T[d][r] = W_UV[d][c] o_lat^T[c][r]: both operands hold
//     consecutive c, so the weights load straight into registers.  Workgroup
//     (h, s) owns output dims 32 s + [0, 32); wave w sums channels [128 w,
//     128 w + 128) and the four partial sums meet in LDS.  The fp32 o_lat is
//     split into bf16 hi + lo (hi = RNE(x), lo = RNE(x - hi)) and both halves go
//     through the matrix core, so the input carries ~16 significant bits into
//     the exact products.
#include "common.hpp"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kAbsRows = 64;              // query rows per workgroup (4 blocks of 16)
constexpr int kAbsSlices = 4;             // workgroups per head
constexpr int kAbsStride = 136;           // halfs per staged W row (128 + 8 pad)

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 lds_tr_b16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
}

// Workgroup (head h, channel slice s, rows [64 g, 64 g + 64)); lane (m, g4) of
// wave w reads, for k-step ks and channel tile t, the transposed 4 x 16 blocks
// so that it holds W_UK[h][32 ks + 8 g4 + j][128 s + 32 w + 16 t + m], j < 8.
__global__ void __launch_bounds__(256)
absorb_q_kernel(const uint16_t* __restrict__ q, int R, int H, const uint16_t* __restrict__ w_uk,
                uint16_t* __restrict__ q_lat) {
  __shared__ __attribute__((aligned(16))) uint16_t stage[kHeadDim * kAbsStride];
  const int h = blockIdx.x;
  const int cs = 128 * blockIdx.y;
  const int r0 = blockIdx.z * kAbsRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const uint16_t* wh = w_uk + (int64_t)h * kHeadDim * kLatent + cs;

  // stage the slice: 128 rows x 256 B, 16 bytes per thread and load
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 16 * i + (tid >> 4);
    v[i] = *reinterpret_cast<const uint4*>(wh + (int64_t)row * kLatent + 8 * (tid & 15));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 16 * i + (tid >> 4);
    *reinterpret_cast<uint4*>(stage + row * kAbsStride + 8 * (tid & 15)) = v[i];
  }
  __syncthreads();

  f32x4 acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kHeadDim / 32; ++ks) {
    // B operands: the query rows of each 16-row block, d = 32 ks + 8 g .. + 7
    bf16x8 qb[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = r0 + 16 * rb + m;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (r < R) x = *reinterpret_cast<const uint4*>(q + ((int64_t)r * H + h) * kHeadDim + 32 * ks + 8 * g);
      qb[rb] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* p = stage + (32 * ks + 8 * g + (m >> 2)) * kAbsStride + 32 * wave + 16 * t + 4 * (m & 3);
      const s16x4 lo = lds_tr_b16(p);
      const s16x4 hi = lds_tr_b16(p + 4 * kAbsStride);
      const short w8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, w8);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb][t] = mfma_bf16(a, qb[rb], acc[rb][t]);
    }
  }
  // C^T[16 t + 4 g + i][row m] -> q_lat[row][h][cs + 32 w + 16 t + 4 g + i], RNE to bf16
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int r = r0 + 16 * rb + m;
    if (r >= R) continue;
    uint16_t* dst = q_lat + ((int64_t)r * H + h) * kLatent + cs + 32 * wave + 4 * g;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 c = acc[rb][t];
      const __bf16 b4[4] = {(__bf16)c[0], (__bf16)c[1], (__bf16)c[2], (__bf16)c[3]};
      *reinterpret_cast<uint2*>(dst + 16 * t) = __builtin_bit_cast(uint2, b4);
    }
  }
}

// Workgroup (head h, dim slice s, rows [64 g, 64 g + 64)): output dims 32 s +
// [0, 32) in two 16-d tiles.  Wave w keeps the A operands of its channel range
// in registers: lane (m, g4) holds W_UV[h][32 s + 16 dt + m][128 w + 32 ks + 8 g4
// .. + 7], ks < 4; the partial sums of the four waves are added through LDS.
__global__ void __launch_bounds__(256)
unabsorb_o_kernel(const float* __restrict__ o_lat, int R, int H, const uint16_t* __restrict__ w_uv,
                  float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) f32x4 red[4][4][2][64];     // wave, row block, dim tile, lane
  const int h = blockIdx.x;
  const int d0 = 32 * blockIdx.y;
  const int r0 = blockIdx.z * kAbsRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int c0 = 128 * wave;
  const uint16_t* wh = w_uv + (int64_t)h * kHeadDim * kLatent;

  bf16x8 wa[2][4];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      wa[dt][ks] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(wh + (int64_t)(d0 + 16 * dt + m) * kLatent + c0 + 32 * ks + 8 * g));

  const int n_rb = min(4, (R - r0 + 15) / 16);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb >= n_rb) break;
    const int r = r0 + 16 * rb + m;
    const bool ok = r < R;
    const float* src = o_lat + ((int64_t)(ok ? r : r0) * H + h) * kLatent + c0 + 8 * g;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + 32 * ks);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 32 * ks + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = ok ? x[j] : 0.f;
        const __bf16 hv = (__bf16)v;
        hi[j] = hv;
        lo[j] = (__bf16)(v - (float)hv);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        acc[dt] = mfma_bf16(wa[dt][ks], hi, acc[dt]);
        acc[dt] = mfma_bf16(wa[dt][ks], lo, acc[dt]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) red[wave][rb][dt][lane] = acc[dt];
  }
  __syncthreads();
  // wave w adds the four partials of row block w: C^T[16 dt + 4 g + i][row m]
  // -> out[row][h][d0 + 16 dt + 4 g + i]
  const int rb = wave;
  if (rb >= n_rb) return;
  const int r = r0 + 16 * rb + m;
  if (r >= R) return;
  float* dst = out + ((int64_t)r * H + h) * kHeadDim + d0 + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    f32x4 v = red[0][rb][dt][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[w][rb][dt][lane];
    *reinterpret_cast<f32x4*>(dst + 16 * dt) = v;
  }
}

}  // namespace csa2

using namespace csa2;

extern "C" csa2_status csa2_absorb_q(const uint16_t* q, int32_t R, int32_t H, int32_t D, const uint16_t* w_uk,
                                     uint16_t* q_lat, void* stream) {
  if (R < 0 || H <= 0) return CSA2_EINVAL;
  if (D != kHeadDim) return CSA2_ESHAPE;
  if (R == 0) return CSA2_OK;
  if (!q || !w_uk || !q_lat) return CSA2_EINVAL;
  if (H > 65535) return CSA2_ESHAPE;
  if (!aligned(q, 16) || !aligned(w_uk, 16) || !aligned(q_lat, 16)) return CSA2_EALIGN;
  if (ceil_div(R, kAbsRows) > 65535) return CSA2_ESHAPE;
  const dim3 grid(H, kAbsSlices, ceil_div(R, kAbsRows));
  absorb_q_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(q, R, H, w_uk, q_lat);
  return launch_status();
}

extern "C" csa2_status csa2_unabsorb_o(const float* o_lat, int32_t R, int32_t H, int32_t D, const uint16_t* w_uv,
                                       float* out, void* stream) {
  if (R < 0 || H <= 0) return CSA2_EINVAL;
  if (D != kHeadDim) return CSA2_ESHAPE;
  if (R == 0) return CSA2_OK;
  if (!o_lat || !w_uv || !out) return CSA2_EINVAL;
  if (H > 65535) return CSA2_ESHAPE;
  if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return CSA2_EALIGN;
  if (ceil_div(R, kAbsRows) > 65535) return CSA2_ESHAPE;
  const dim3 grid(H, kAbsSlices, ceil_div(R, kAbsRows));
  unabsorb_o_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(o_lat, R, H, w_uv, out);
  return launch_status();
}
