// Sparse attention over the FP4 cache and sliding-window attention with
// log-sum-exp merge (HN summary key points: local sliding window plus global
// sparse retrieval over the shared main KV; MarkTechPost retelling, paragraph
// 2: a 128-token window in every layer).
//
// Absorbed multi-head latent attention: every head of a row attends over the
// same 512-channel latent rows, used as key and as value.
//
// Work split (split-K, "flash-decoding"): a workgroup owns one query row, a
// chunk of key tiles and NW*16 heads (one wave per 16 heads).  Per 32-key tile:
//   1. gather: each thread fetches 32 bytes of codes + 4 scale bytes of one
//      key (16-byte loads), or 128 bytes of a bf16 window row, for the NEXT
//      tile while the current one is computed;
//   2. dequantise to fp16 (exact: E2M1 x E4M3 has <= 6 significant bits and
//      lies in [2^-10, 2688]) into LDS twice: key-major Xs[key][channel] and
//      channel-major Xt[channel][key];
//   3. S^T[key][head] = X . Q^T on v_mfma_f32_16x16x32_f16 (A = Xs rows,
//      B = the wave's queries held in registers as fp16);
//   4. online softmax in the exp2 domain: each lane owns one head's column,
//      so the row max / sum need two cross-lane steps;
//   5. O^T[channel][head] += Xt . P^T on the same MFMA (A = Xt rows, B = P
//      straight from the softmax registers), fp32 accumulators in VGPRs.
// The chunk's unnormalised O, running max m and sum l go to the workspace; a
// combine kernel merges chunks (and, for the window call, the sparse result)
// into o and lse.
#include <type_traits>

#include "common.hpp"

namespace csa2 {

constexpr int kKT = 32;                  // keys per tile
constexpr int kXsStride = kLatent + 8;   // halfs per key row of Xs
constexpr int kXtStride = kKT + 8;       // halfs per channel row of Xt
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 E2M1 nibbles (one code dword, channel 2j in the low nibble of byte j) ->
// 4 dwords of fp16 pairs, multiplied by the block scale (fp16 pair).
// The fp16 high byte of each E2M1 magnitude {0,.5,1,1.5,2,3,4,6} is
// {00,38,3C,3E,40,42,44,46} and its low byte is 0, so a byte permute does the
// table lookup.
__device__ __forceinline__ void fp4x8_to_f16(uint32_t d, f16x2 s2, uint32_t* out) {
  const uint32_t lut_lo = 0x3E3C3800u, lut_hi = 0x46444240u;
  uint32_t me = d & 0x07070707u;
  uint32_t mo = (d >> 4) & 0x07070707u;
  uint32_t he = __builtin_amdgcn_perm(lut_hi, lut_lo, me) | ((d << 4) & 0x80808080u);
  uint32_t ho = __builtin_amdgcn_perm(lut_hi, lut_lo, mo) | (d & 0x80808080u);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t sel = 0x0Cu | ((uint32_t)k << 8) | (0x0Cu << 16) | ((uint32_t)(4 + k) << 24);
    uint32_t v = __builtin_amdgcn_perm(ho, he, sel);
    f16x2 h = __builtin_bit_cast(f16x2, v) * s2;
    out[k] = __builtin_bit_cast(uint32_t, h);
  }
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  float a = __uint_as_float(w << 16), b = __uint_as_float(w & 0xFFFF0000u);
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// raw global data of one (key, 64-channel part) item
struct RawFp4 {
  uint4 c0, c1;
  uint32_t sc;
  int valid;
};
struct RawBf16 {
  uint4 v[8];
  int valid;
};

template <int NW, bool kWindow>
struct Loader {
  static constexpr int kThreads = NW * 64;
  static constexpr int kTotal = kKT * 8;                  // (key, 64-channel part) items per tile
  static constexpr int kItems = (kTotal + kThreads - 1) / kThreads;    // items per thread
  using Raw = typename std::conditional<kWindow, RawBf16, RawFp4>::type;
};

template <int NW, bool kWindow>
__global__ void __launch_bounds__(NW * 64)
attn_partial_kernel(const uint16_t* __restrict__ q_lat, int H,
                    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                    const uint16_t* __restrict__ swa, int S, int64_t T, const int32_t* __restrict__ row_seq,
                    const int32_t* __restrict__ idx, int K,
                    const int32_t* __restrict__ swa_start, const int32_t* __restrict__ swa_len,
                    float scale_log2, int tiles_per_chunk, int n_chunks,
                    float* __restrict__ o_part, float* __restrict__ ml_part) {
  using L = Loader<NW, kWindow>;
  using Raw = typename L::Raw;
  __shared__ __attribute__((aligned(16))) _Float16 xs[kKT * kXsStride];
  __shared__ __attribute__((aligned(16))) _Float16 xt[kLatent * kXtStride];
  __shared__ int s_valid[kKT];

  const int chunk = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.z * (NW * 16) + wave * 16 + n16;   // this lane's head (column)
  const int seq = row_seq ? row_seq[r] : r;

  // key range of this chunk
  int n_keys, k_base, w_start = 0;
  if (kWindow) {
    int st = swa_start[r], ln = swa_len[r];
    bool ok = st >= 0 && ln >= 0 && ln <= kWindowMax && (int64_t)st + ln <= S;
    n_keys = ok ? ln : 0;
    w_start = ok ? st : 0;
  } else {
    n_keys = K;
  }
  k_base = chunk * tiles_per_chunk * kKT;
  const int k_end = min(n_keys, k_base + tiles_per_chunk * kKT);
  const int n_tiles = k_end > k_base ? (k_end - k_base + kKT - 1) / kKT : 0;

  // queries: B operand of S^T = X . Q^T; k-step ks holds channels 32ks + 8g + [0,8)
  f16x8 qreg[16];
  {
    const uint16_t* qrow = q_lat + ((int64_t)r * H + h) * kLatent;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
      uint32_t w[4] = {bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
      qreg[ks] = __builtin_bit_cast(f16x8, w);
    }
  }

  f32x4 o_acc[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) o_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  Raw raw[L::kItems];

  auto load_tile = [&](int tile) {
    const int k0 = k_base + tile * kKT;
#pragma unroll
    for (int it = 0; it < L::kItems; ++it) {
      const int item = tid + it * L::kThreads;
      if (item >= L::kTotal) break;
      const int key = item >> 3, part = item & 7;
      const int kk = k0 + key;
      if constexpr (kWindow) {
        bool ok = kk < k_end;
        raw[it].valid = ok;
        if (ok) {
          const uint4* p = reinterpret_cast<const uint4*>(
              swa + ((int64_t)seq * S + w_start + kk) * kLatent + 64 * part);
#pragma unroll
          for (int j = 0; j < 8; ++j) raw[it].v[j] = p[j];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) raw[it].v[j] = make_uint4(0, 0, 0, 0);
        }
      } else {
        int pos = kk < k_end ? idx[(int64_t)r * K + kk] : -1;
        bool ok = pos >= 0 && pos < T;
        raw[it].valid = ok;
        if (ok) {
          const int64_t row = (int64_t)seq * T + pos;
          const uint4* pc = reinterpret_cast<const uint4*>(codes + row * kCodesRow + 32 * part);
          raw[it].c0 = pc[0];
          raw[it].c1 = pc[1];
          raw[it].sc = *reinterpret_cast<const uint32_t*>(scales + row * kScalesRow + 4 * part);
        } else {
          raw[it].c0 = make_uint4(0, 0, 0, 0);
          raw[it].c1 = make_uint4(0, 0, 0, 0);
          raw[it].sc = 0;
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < L::kItems; ++it) {
      const int item = tid + it * L::kThreads;
      if (item >= L::kTotal) break;
      const int key = item >> 3, part = item & 7;
      uint32_t hv[32];                   // 64 fp16 values of this item
      if constexpr (kWindow) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          hv[4 * j + 0] = bf16x2_to_f16x2(raw[it].v[j].x);
          hv[4 * j + 1] = bf16x2_to_f16x2(raw[it].v[j].y);
          hv[4 * j + 2] = bf16x2_to_f16x2(raw[it].v[j].z);
          hv[4 * j + 3] = bf16x2_to_f16x2(raw[it].v[j].w);
        }
      } else {
        uint32_t cw[8] = {raw[it].c0.x, raw[it].c0.y, raw[it].c0.z, raw[it].c0.w,
                          raw[it].c1.x, raw[it].c1.y, raw[it].c1.z, raw[it].c1.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {         // 4 scale blocks of 16 channels = 2 code dwords each
          float sf = e4m3_to_f32((raw[it].sc >> (8 * b)) & 0xFFu);
          f16x2 s2 = {(_Float16)sf, (_Float16)sf};
          fp4x8_to_f16(cw[2 * b], s2, &hv[8 * b]);
          fp4x8_to_f16(cw[2 * b + 1], s2, &hv[8 * b + 4]);
        }
      }
      // key-major copy: 64 halfs = 8 x 16 bytes
      uint4* dst = reinterpret_cast<uint4*>(&xs[key * kXsStride + 64 * part]);
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = make_uint4(hv[4 * j], hv[4 * j + 1], hv[4 * j + 2], hv[4 * j + 3]);
      // channel-major copy
      uint16_t* xt16 = reinterpret_cast<uint16_t*>(xt);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        xt16[(64 * part + 2 * j) * kXtStride + key] = (uint16_t)(hv[j] & 0xFFFFu);
        xt16[(64 * part + 2 * j + 1) * kXtStride + key] = (uint16_t)(hv[j] >> 16);
      }
      if (part == 0) s_valid[key] = raw[it].valid;
    }
  };

  if (n_tiles > 0) load_tile(0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    __syncthreads();                 // previous tile's LDS reads are done
    store_tile();
    __syncthreads();
    if (tile + 1 < n_tiles) load_tile(tile + 1);   // in flight during the math below

    // ---- S^T = X . Q^T : two 16-key M-tiles
    f32x4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const _Float16* xrow = &xs[(16 * mt + n16) * kXsStride + 8 * g];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        f16x8 a = *reinterpret_cast<const f16x8*>(xrow + 32 * ks);
        acc = mfma16(a, qreg[ks], acc);
      }
      sacc[mt] = acc;
    }
    // ---- online softmax (lane column = head h; rows = keys 16mt + 4g + i)
    float s[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int key = 16 * mt + 4 * g + i;
        float v = s_valid[key] ? sacc[mt][i] * scale_log2 : -__builtin_inff();
        s[4 * mt + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool live = m_new != -__builtin_inff();
    const float alpha = live ? exp2f(m_run - m_new) : 1.f;
    float psum = 0.f;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = live ? exp2f(s[j] - m_new) : 0.f;
      psum += p[j];
    }
    psum += shfl_xor_f(psum, 16);
    psum += shfl_xor_f(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int t = 0; t < 32; ++t) o_acc[t] *= alpha;
    }
    // ---- O^T += Xt . P^T ; slot j<4 -> key 4g+j, j>=4 -> key 16+4g+(j-4)
    f16x8 pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[j] = (_Float16)p[j];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const _Float16* xr = &xt[(16 * t + n16) * kXtStride];
      f16x4 a0 = *reinterpret_cast<const f16x4*>(xr + 4 * g);
      f16x4 a1 = *reinterpret_cast<const f16x4*>(xr + 16 + 4 * g);
      f16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      o_acc[t] = mfma16(a, pb, o_acc[t]);
    }
  }

  // ---- write this chunk's partial: O^T lane holds channels 16t + 4g + i of head h
  const int64_t prow = ((int64_t)r * n_chunks + chunk) * H + h;
  float* op = o_part + prow * kLatent;
#pragma unroll
  for (int t = 0; t < 32; ++t)
    *reinterpret_cast<f32x4*>(op + 16 * t + 4 * g) = o_acc[t];
  if (g == 0) {
    ml_part[prow * 2 + 0] = m_run;
    ml_part[prow * 2 + 1] = l_run;
  }
}

// Merge the chunk partials of each (row, head), optionally with a finished
// prior result (o_prev normalised, lse_prev natural log), into o and lse.
__global__ void __launch_bounds__(128)
attn_combine_kernel(const float* __restrict__ o_part, const float* __restrict__ ml_part, int n_chunks, int H,
                    const float* __restrict__ o_prev, const float* __restrict__ lse_prev,
                    float* __restrict__ o_out, float* __restrict__ lse_out) {
  const int h = blockIdx.x, r = blockIdx.y;
  const int c4 = threadIdx.x * 4;
  const int64_t base = ((int64_t)r * n_chunks) * H + h;       // + chunk * H
  float M = -__builtin_inff();
  for (int c = 0; c < n_chunks; ++c) {
    float m = ml_part[(base + (int64_t)c * H) * 2];
    float l = ml_part[(base + (int64_t)c * H) * 2 + 1];
    if (l > 0.f) M = fmaxf(M, m);
  }
  float mp = -__builtin_inff();
  if (lse_prev) {
    mp = lse_prev[(int64_t)r * H + h] * kLog2e;
    M = fmaxf(M, mp);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Lsum = 0.f;
  if (M != -__builtin_inff()) {
    for (int c = 0; c < n_chunks; ++c) {
      float m = ml_part[(base + (int64_t)c * H) * 2];
      float l = ml_part[(base + (int64_t)c * H) * 2 + 1];
      if (!(l > 0.f)) continue;
      float w = exp2f(m - M);
      Lsum += l * w;
      f32x4 v = *reinterpret_cast<const f32x4*>(o_part + (base + (int64_t)c * H) * kLatent + c4);
      acc += v * w;
    }
    if (lse_prev && mp != -__builtin_inff()) {
      float w = exp2f(mp - M);
      Lsum += w;
      f32x4 v = *reinterpret_cast<const f32x4*>(o_prev + ((int64_t)r * H + h) * kLatent + c4);
      acc += v * w;
    }
  }
  f32x4 res = Lsum > 0.f ? acc * (1.f / Lsum) : f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();                 // o_out / lse_out may alias o_prev / lse_prev
  *reinterpret_cast<f32x4*>(o_out + ((int64_t)r * H + h) * kLatent + c4) = res;
  if (lse_out && threadIdx.x == 0)
    lse_out[(int64_t)r * H + h] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct SparsePlan {
  int tiles_per_chunk;
  int n_chunks;
};

static SparsePlan sparse_plan(int32_t R, int32_t K) {
  int tiles = (K + kKT - 1) / kKT;
  if (tiles < 1) tiles = 1;
  // about 512 workgroups in total, at least 4 tiles per chunk so that the
  // partial outputs stay small next to the gathered rows
  int want = (512 + R - 1) / R;
  int tpc = (tiles + want - 1) / want;
  if (tpc < 4) tpc = 4;
  if (tpc > tiles) tpc = tiles;
  SparsePlan p{tpc, (tiles + tpc - 1) / tpc};
  return p;
}

static size_t partial_bytes(int32_t R, int32_t H, int n_chunks, size_t* off_ml) {
  size_t o = align_up((size_t)R * n_chunks * H * kLatent * sizeof(float), 256);
  size_t ml = align_up((size_t)R * n_chunks * H * 2 * sizeof(float), 256);
  if (off_ml) *off_ml = o;
  return o + ml;
}

static bool heads_ok(int32_t H) { return H == 16 || H == 32 || H == 48 || H == 64; }

template <bool kWindow>
static void launch_partial(int NW, dim3 grid, hipStream_t s, const uint16_t* q_lat, int H, const uint8_t* codes,
                           const uint8_t* scales, const uint16_t* swa, int S, int64_t T, const int32_t* row_seq,
                           const int32_t* idx, int K, const int32_t* swa_start, const int32_t* swa_len,
                           float scale_log2, int tpc, int n_chunks, float* o_part, float* ml_part) {
#define CSA2_LAUNCH(NWV)                                                                                     \
  attn_partial_kernel<NWV, kWindow><<<grid, NWV * 64, 0, s>>>(q_lat, H, codes, scales, swa, S, T, row_seq, \
                                                             idx, K, swa_start, swa_len, scale_log2, tpc,   \
                                                             n_chunks, o_part, ml_part)
  switch (NW) {
    case 1: CSA2_LAUNCH(1); break;
    case 2: CSA2_LAUNCH(2); break;
    case 3: CSA2_LAUNCH(3); break;
    default: CSA2_LAUNCH(4); break;
  }
#undef CSA2_LAUNCH
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_sparse_decode_workspace_size(int32_t R, int32_t H, int32_t K) {
  if (R <= 0 || H <= 0 || K <= 0) return 0;
  SparsePlan p = sparse_plan(R, K);
  return partial_bytes(R, H, p.n_chunks, nullptr);
}

extern "C" csa2_status csa2_sparse_decode(const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* codes,
                                          const uint8_t* scales, int32_t B, int64_t T, const int32_t* row_seq,
                                          const int32_t* idx, int32_t K, float softmax_scale, float* o,
                                          float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_lat || !codes || !scales || !idx || !o || !lse) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0 || K <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (!heads_ok(H)) return CSA2_ESHAPE;
  if (T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_lat, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(idx, 4) ||
      !aligned(o, 16) || !aligned(lse, 4))
    return CSA2_EALIGN;
  SparsePlan p = sparse_plan(R, K);
  size_t off_ml;
  size_t need = partial_bytes(R, H, p.n_chunks, &off_ml);
  if (!workspace || workspace_bytes < need) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  float* o_part = static_cast<float*>(workspace);
  float* ml_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + off_ml);
  hipStream_t s = (hipStream_t)stream;
  const int NW = H / 16;
  dim3 grid(p.n_chunks, R, 1);
  launch_partial<false>(NW, grid, s, q_lat, H, codes, scales, nullptr, 0, T, row_seq, idx, K, nullptr, nullptr,
                        softmax_scale * kLog2e, p.tiles_per_chunk, p.n_chunks, o_part, ml_part);
  attn_combine_kernel<<<dim3(H, R), 128, 0, s>>>(o_part, ml_part, p.n_chunks, H, nullptr, nullptr, o, lse);
  return launch_status();
}

extern "C" size_t csa2_swa_merge_workspace_size(int32_t R, int32_t H) {
  if (R <= 0 || H <= 0) return 0;
  return partial_bytes(R, H, kWindowMax / kKT, nullptr);
}

extern "C" csa2_status csa2_swa_merge(const uint16_t* q_lat, int32_t R, int32_t H, const uint16_t* swa, int32_t B,
                                      int32_t S, const int32_t* row_seq, const int32_t* swa_start,
                                      const int32_t* swa_len, float softmax_scale, const float* o_sparse,
                                      const float* lse_sparse, float* o_out, float* lse_out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!q_lat || !swa || !swa_start || !swa_len || !o_out) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || S <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if ((o_sparse == nullptr) != (lse_sparse == nullptr)) return CSA2_EINVAL;
  if (!heads_ok(H)) return CSA2_ESHAPE;
  if (!aligned(q_lat, 16) || !aligned(swa, 16) || !aligned(o_out, 16) || (o_sparse && !aligned(o_sparse, 16)))
    return CSA2_EALIGN;
  const int n_chunks = kWindowMax / kKT;
  size_t off_ml;
  size_t need = partial_bytes(R, H, n_chunks, &off_ml);
  if (!workspace || workspace_bytes < need) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  float* o_part = static_cast<float*>(workspace);
  float* ml_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + off_ml);
  hipStream_t s = (hipStream_t)stream;
  const int NW = H / 16;
  dim3 grid(n_chunks, R, 1);
  launch_partial<true>(NW, grid, s, q_lat, H, nullptr, nullptr, swa, S, 0, row_seq, nullptr, 0, swa_start, swa_len,
                       softmax_scale * kLog2e, 1, n_chunks, o_part, ml_part);
  attn_combine_kernel<<<dim3(H, R), 128, 0, s>>>(o_part, ml_part, n_chunks, H, o_sparse, lse_sparse, o_out, lse_out);
  return launch_status();
}
