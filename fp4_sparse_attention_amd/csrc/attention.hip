// Sparse attention over the FP4 cache and sliding-window attention with
// log-sum-exp merge (HN summary key points: local sliding window plus global
// sparse retrieval over the shared main KV; MarkTechPost retelling, paragraph
// 2: a 128-token window in every layer).
//
// Absorbed multi-head latent attention: every head of a row attends over the
// same 512-channel latent rows, used as key and as value.
//
// Work split (split-K): a workgroup of four waves owns one query row and one
// chunk of keys (a run of 32-key tiles from idx, or one 32-row tile of the row's window), for
// all H <= 64 heads.  Wave w owns latent channels [128w, 128w+128):
//   1. gather: lane (m = l%16, g = l/16) loads 16 code bytes + 2 scale bytes
//      (32 channels) of keys m and 16+m of the tile -- each FP4 element is
//      fetched and dequantised by exactly one lane; the next tile's loads are
//      in flight during the current tile's math;
//   2. dequantise in registers (v_cvt_scalef32_pk_f16_fp4 with unit scale,
//      times the E4M3 block scale in f16: exact, <= 6 significant bits in
//      [2^-10, 2688]) straight into the A operands of
//      v_mfma_f32_16x16x32_f16, and store the slice key-major in LDS;
//   3. partial scores S^T[key][head] over the wave's 128 channels (B = the
//      wave's slice of the queries, kept in registers);
//   4. the four partials meet in LDS; wave w sums them for heads [16w, 16w+16)
//      and runs the online softmax in the exp2 domain (one head per lane
//      column, two cross-lane steps), publishing P (f16) and the rescale factors;
//   5. O^T[channel][head] += X^T P^T for the wave's channels: the A operand is
//      read from the key-major slice with ds_read_b64_tr_b16 (gfx950 LDS
//      transpose load), B = P from LDS; fp32 accumulators stay in VGPRs.
// The chunk's unnormalised O, running max m and sum l go to the workspace; a
// combine kernel merges the chunks (and, for a window merge, the sparse
// result) into o and lse.  When a row has one chunk and no prior result (enough
// rows to fill the chip, e.g. chunked prefill), the chunk kernel normalises and
// writes o and lse itself, with the combine's arithmetic for one chunk.
#include <type_traits>

#include "internal.hpp"

namespace csa2 {

constexpr int kKT = 32;                  // keys per tile
constexpr int kXwStride = 144;           // halfs per key row of a wave's slice (128 + 16 pad)
constexpr int kSStride = 36;             // floats per head row of a partial-score tile
constexpr int kPStride = 40;             // halfs per head row of P
constexpr int kMaxChunkTiles = 64;       // tiles per chunk at most
constexpr int kMaxChunkKeys = kMaxChunkTiles * kKT;
constexpr int kWindowChunks = kWindowMax / kKT;   // one-tile chunks covering the longest window
constexpr float kRescaleSlack = 8.0f;    // keep the reference max until exceeded by 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 E2M1 nibbles (one code dword; channel 2j in the low nibble of byte j) times
// the block scale -> f16x8, exact.
__device__ __forceinline__ f16x8 fp4x8_to_f16(uint32_t d, f16x2 s2) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * s2;
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * s2;
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * s2;
  f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * s2;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  float a = __uint_as_float(w << 16), b = __uint_as_float(w & 0xFFFF0000u);
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ f16x8 bf16x8_to_f16(uint4 v) {
  uint32_t w[4] = {bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
  return __builtin_bit_cast(f16x8, w);
}

__device__ __forceinline__ f16x4 lds_tr16(const _Float16* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(f16x4, v);
}

constexpr int kMaxLayers = 8;
constexpr int kPrefetch = 4;             // sparse tiles whose gathers are in flight ahead of the math (4 vs 2: -1.3 us on the 8 x 1M stack)

// One launch covers L layers.  Layer l has its own queries, window rows and
// outputs, and reads the index slice at idx + idx_off[l] (layers may share one).
// Each (layer, row) splits its keys into n_chunks chunks: chunk c takes the
// window tiles [c wpc, (c+1) wpc) (tile w: rows [32w, 32w+32) of the window)
// and the sparse tiles [c spc, (c+1) spc).  Window tiles go first; the loads of
// the first one are issued at the start of the workgroup.
struct AttnArgs {
  const uint16_t* q_lat;          // bf16 [L][R][H][512]
  int R, H, L, head_groups;
  const uint8_t* codes;           // [B][T][256]
  const uint8_t* scales;          // [B][T][32]
  int64_t T;
  const int32_t* row_seq;         // [R] or null
  const int32_t* idx;             // index slices [.][R][K]
  int64_t idx_off[kMaxLayers];    // element offset of layer l's slice
  int K;
  int n_sparse_tiles;             // ceil(K / 32), 0 without sparse keys
  int n_window_tiles;             // tiles covering the longest window, 0 without a window
  int window_per_chunk;           // window tiles per chunk
  int sparse_per_chunk;           // sparse tiles per chunk
  int n_chunks;
  const uint16_t* swa;            // bf16 [L][B][S][512]
  int B, S;
  const int32_t* swa_start;       // [L][R]
  const int32_t* swa_len;         // [L][R]
  float scale_log2;               // softmax scale * log2(e)
  float* o_part;                  // [L][R][n_chunks][H][512]
  float* ml_part;                 // [L][R][n_chunks][H][2]
  float* o_out;                   // one chunk and no prior: the final o [L][R][H][512] (null: partials)
  float* lse_out;                 // and lse [L][R][H] (may be null then)
  PageMap pm;                     // codes / scales as page pools (table null: [B][T] rows)
};

// raw FP4 data of the lane's two keys for one tile (gathered kPrefetch tiles ahead)
struct RawTile {
  uint4 v[2];         // 16 code bytes (32 channels) per key
  uint32_t sc[2];     // 2 scale bytes per key
  int valid[2];
};

template <int NT>
__global__ void __launch_bounds__(256, 2)
attn_chunk_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 xw[4 * kKT * kXwStride];
  __shared__ __attribute__((aligned(16))) float sp[4 * NT * 16 * kSStride];
  __shared__ __attribute__((aligned(16))) _Float16 pp[NT * 16 * kPStride];
  __shared__ float s_alpha[NT * 16];
  __shared__ float s_inv_l[NT * 16];
  __shared__ int s_valid[kKT];
  __shared__ int s_pos[kMaxChunkKeys];        // this chunk's cache positions (-1: skip)

  const int chunk = blockIdx.x;
  const int r = blockIdx.y;
  const int layer = blockIdx.z / a.head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;
  const int g = lane >> 4;
  const int H = a.H;
  const int hbase = (blockIdx.z % a.head_groups) * NT * 16;      // this workgroup's first head
  const int seq = a.row_seq ? a.row_seq[r] : r;
  const int cbase = 128 * wave;                                   // this wave's channel slice

  // this chunk's tiles: window tiles [w0, w0 + n_wt), then sparse tiles [sp0, sp0 + n_sp)
  const int w0 = chunk * a.window_per_chunk;
  const int n_wt = max(0, min(a.n_window_tiles, w0 + a.window_per_chunk) - w0);
  const int sp0 = chunk * a.sparse_per_chunk;
  const int n_sp = max(0, min(a.n_sparse_tiles, sp0 + a.sparse_per_chunk) - sp0);
  const int k0 = sp0 * kKT;
  const int k1 = min(a.K, (sp0 + n_sp) * kKT);

  // window rows of tile w: lane (m, g) takes channels cbase + 32g + [0, 32) of rows 32w + 16mt + m
  uint4 wv[2][4];
  int wvalid[2] = {0, 0};
  int w_st = 0, w_ln = 0;
  const uint16_t* swa_l = nullptr;
  if (n_wt > 0) {
    const int st = a.swa_start[layer * a.R + r], ln = a.swa_len[layer * a.R + r];
    const bool ok = st >= 0 && ln >= 0 && ln <= kWindowMax && (int64_t)st + ln <= a.S;
    w_st = ok ? st : 0;
    w_ln = ok ? ln : 0;
    swa_l = a.swa + (int64_t)layer * a.B * a.S * kLatent;
  }
  auto load_window = [&](int w) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int kk = w * kKT + 16 * mt + m;
      wvalid[mt] = kk < w_ln;
      const uint4* p = reinterpret_cast<const uint4*>(swa_l + ((int64_t)seq * a.S + (wvalid[mt] ? w_st + kk : 0)) *
                                                      kLatent + cbase + 32 * g);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) wv[mt][ks] = wvalid[mt] ? p[ks] : make_uint4(0, 0, 0, 0);
    }
  };
  if (n_wt > 0) load_window(w0);

  // queries: B operand of S^T = X . Q^T; k-step ks holds channels cbase + 32g + 8ks + [0, 8)
  const uint16_t* q_l = a.q_lat + (int64_t)layer * a.R * H * kLatent;
  f16x8 qb[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint16_t* qrow = q_l + ((int64_t)r * H + hbase + 16 * nt + m) * kLatent + cbase + 32 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[nt][ks] = bf16x8_to_f16(*reinterpret_cast<const uint4*>(qrow + 8 * ks));
  }

  f32x4 oacc[8][NT];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  // positions of this chunk's sparse keys, staged once so that the gathers
  // below do not wait on dependent index loads
  if (n_sp > 0) {
    const int32_t* idx_row = a.idx + a.idx_off[layer] + (int64_t)r * a.K;
    for (int i = tid; i < n_sp * kKT; i += 256) {
      const int kk = k0 + i;
      const int pos = kk < k1 ? idx_row[kk] : -1;
      s_pos[i] = (pos >= 0 && pos < a.T) ? pos : -1;
    }
    __syncthreads();
  }

  // gather the FP4 codes + scales of sparse tile j's keys into a register buffer
  auto load_tile = [&](RawTile& raw, int j) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int pos = s_pos[j * kKT + 16 * mt + m];
      const int64_t row = pos >= 0 ? phys_row(a.pm, seq, a.T, pos) : -1;
      const bool ok = row >= 0;
      raw.valid[mt] = ok;
      if (ok) {
        raw.v[mt] = *reinterpret_cast<const uint4*>(a.codes + row * kCodesRow + 64 * wave + 16 * g);
        raw.sc[mt] = *reinterpret_cast<const uint16_t*>(a.scales + row * kScalesRow + 8 * wave + 2 * g);
      } else {
        raw.v[mt] = make_uint4(0, 0, 0, 0);
        raw.sc[mt] = 0;
      }
    }
  };

  _Float16* xmine = xw + wave * kKT * kXwStride;
  float* spmine = sp + wave * NT * 16 * kSStride;
  const float neg_inf = -__builtin_inff();

  // one tile: the window tile (win) or sparse tile j, whose buffer is refilled with j + 2
  auto process = [&](RawTile& raw, bool win, int j) {
    // ---- per 16-key half-tile: dequantise this wave's slice into A operands,
    //      store it key-major in LDS, and form the partial scores
    //      S^T[16mt + 4g + i][16nt + m] over the wave's 128 channels
    int valid_mt[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f16x8 xa[4];
      if (!win) {
        const uint32_t cw[4] = {raw.v[mt].x, raw.v[mt].y, raw.v[mt].z, raw.v[mt].w};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const float sf = e4m3_to_f32((raw.sc[mt] >> (8 * (ks >> 1))) & 0xFFu);
          const f16x2 s2 = {(_Float16)sf, (_Float16)sf};
          xa[ks] = fp4x8_to_f16(cw[ks], s2);
        }
        valid_mt[mt] = raw.valid[mt];
      } else {
        // window rows: bf16 -> f16
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) xa[ks] = bf16x8_to_f16(wv[mt][ks]);
        valid_mt[mt] = wvalid[mt];
      }
      f16x8* dst = reinterpret_cast<f16x8*>(xmine + (16 * mt + m) * kXwStride + 32 * g);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dst[ks] = xa[ks];
      f32x4 sacc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[nt] = mfma16(xa[ks], qb[nt][ks], sacc[nt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4*>(spmine + (16 * nt + m) * kSStride + 16 * mt + 4 * g) = sacc[nt];
      if (!win && mt == 1 && j + kPrefetch < n_sp) load_tile(raw, j + kPrefetch);   // buffer free: refill it
    }
    if (wave == 0 && g == 0) {
      s_valid[m] = valid_mt[0];
      s_valid[16 + m] = valid_mt[1];
    }
    __syncthreads();

    // ---- softmax for heads [16w, 16w+16): lane (m, g) owns head 16w+m, keys 8g + [0, 8)
    if (wave < NT) {
      float s[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float* src = sp + w2 * NT * 16 * kSStride + (16 * wave + m) * kSStride + 8 * g;
        f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
        f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { s[q] += v0[q]; s[4 + q] += v1[q]; }
      }
      float mx = neg_inf;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        s[q] = s_valid[8 * g + q] ? s[q] * a.scale_log2 : neg_inf;
        mx = fmaxf(mx, s[q]);
      }
      mx = xor32_max(xor16_max(mx));
      // P = 2^(s - m_ref) stays <= 2^8 in f16; m_ref moves only past that slack
      const float m_new = (mx > m_run + kRescaleSlack) ? mx : m_run;
      const bool live = m_new != neg_inf;
      const float alpha = live ? exp2f(m_run - m_new) : 1.f;
      float psum = 0.f;
      f16x8 ph;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float pj = live ? exp2f(s[q] - m_new) : 0.f;
        psum += pj;
        ph[q] = (_Float16)pj;
      }
      psum = xor32_sum(xor16_sum(psum));
      l_run = l_run * alpha + psum;
      m_run = m_new;
      *reinterpret_cast<f16x8*>(pp + (16 * wave + m) * kPStride + 8 * g) = ph;
      if (g == 0) s_alpha[16 * wave + m] = alpha;
    }
    __syncthreads();

    // ---- rescale and accumulate O^T[cbase + 16t + 4g + i][16nt + m] += sum_k X[k][.] P[.][k]
    float al[NT];
    bool any_scale = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      al[nt] = s_alpha[16 * nt + m];
      any_scale |= al[nt] != 1.f;
    }
    if (__any(any_scale)) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[t][nt] *= al[nt];
    }
    f16x8 pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pb[nt] = *reinterpret_cast<const f16x8*>(pp + (16 * nt + m) * kPStride + 8 * g);
    // transpose-read rows: source lane m supplies keys 8g + (m>>2) (+4) and channels 16t + 4(m&3) .. +3
    const _Float16* tr0 = xmine + (8 * g + (m >> 2)) * kXwStride + 4 * (m & 3);
    const _Float16* tr1 = tr0 + 4 * kXwStride;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f16x4 lo = lds_tr16(tr0 + 16 * t);
      f16x4 hi = lds_tr16(tr1 + 16 * t);
      f16x8 xt = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[t][nt] = mfma16(xt, pb[nt], oacc[t][nt]);
    }
  };

  RawTile buf[kPrefetch];
#pragma unroll
  for (int b = 0; b < kPrefetch; ++b)
    if (b < n_sp) load_tile(buf[b], b);
  for (int i = 0; i < n_wt; ++i) {
    if (i > 0) load_window(w0 + i);
    process(buf[0], true, -1);
  }
  for (int j = 0; j < n_sp; j += kPrefetch) {
#pragma unroll
    for (int b = 0; b < kPrefetch; ++b)
      if (j + b < n_sp) process(buf[b], false, j + b);
  }

  if (a.o_out) {
    // the row's only chunk and no prior: normalise here, as the combine would for one chunk
    if (wave < NT && g == 0) s_inv_l[16 * wave + m] = l_run > 0.f ? 1.f / l_run : 0.f;
    __syncthreads();
    const int64_t orow = ((int64_t)layer * a.R + r) * H + hbase;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float inv = s_inv_l[16 * nt + m];
      float* op = a.o_out + (orow + 16 * nt + m) * kLatent + cbase + 4 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<f32x4*>(op + 16 * t) = inv > 0.f ? oacc[t][nt] * inv : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (a.lse_out && wave < NT && g == 0)
      a.lse_out[orow + 16 * wave + m] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : neg_inf;
    return;
  }
  // ---- this chunk's partial: unnormalised O, and (m, l) from the softmax owners
  const int64_t prow = (((int64_t)layer * a.R + r) * a.n_chunks + chunk) * H + hbase;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float* op = a.o_part + (prow + 16 * nt + m) * kLatent + cbase + 4 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = oacc[t][nt];
  }
  if (wave < NT && g == 0) {
    a.ml_part[(prow + 16 * wave + m) * 2 + 0] = m_run;
    a.ml_part[(prow + 16 * wave + m) * 2 + 1] = l_run;
  }
}

// Merge the chunk partials of each (row, head), optionally with a finished
// prior result (o_prev normalised, lse_prev natural log), into o and lse.
// Thread t owns channels [4t, 4t+4).  The chunk weights 2^(m_c - M) go through
// LDS in batches of 128 chunks so that every partial-row load of a batch is
// independent of the others (no load waits on the previous chunk's).
constexpr int kCombineThreads = 128;

__device__ __forceinline__ float block_max_128(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(red[0], red[1]);
  __syncthreads();
  return v;
}

__device__ __forceinline__ float block_sum_128(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor_f(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0] + red[1];
  __syncthreads();
  return v;
}

__global__ void __launch_bounds__(kCombineThreads)
attn_combine_kernel(const float* __restrict__ o_part, const float* __restrict__ ml_part, int n_chunks, int R, int H,
                    const float* __restrict__ o_prev, const float* __restrict__ lse_prev,
                    float* __restrict__ o_out, float* __restrict__ lse_out) {
  __shared__ float s_w[kCombineThreads];
  __shared__ float red[2];
  const int h = blockIdx.x, r = blockIdx.y, layer = blockIdx.z;
  const int tid = threadIdx.x;
  const int c4 = tid * 4;
  const int64_t base = (((int64_t)layer * R + r) * n_chunks) * H + h;       // + chunk * H
  const int64_t orow = ((int64_t)layer * R + r) * H + h;                   // output (row, head) of this layer
  const float neg_inf = -__builtin_inff();
  float M = neg_inf;
  for (int c = tid; c < n_chunks; c += kCombineThreads) {
    const float2 ml = *reinterpret_cast<const float2*>(ml_part + (base + (int64_t)c * H) * 2);
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  M = block_max_128(M, red);
  float mp = neg_inf;
  if (lse_prev) {
    mp = lse_prev[orow] * kLog2e;
    M = fmaxf(M, mp);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lpart = 0.f;
  if (M != neg_inf) {
    for (int c0 = 0; c0 < n_chunks; c0 += kCombineThreads) {
      const int c = c0 + tid;
      float w = 0.f;
      if (c < n_chunks) {
        const float2 ml = *reinterpret_cast<const float2*>(ml_part + (base + (int64_t)c * H) * 2);
        if (ml.y > 0.f) {
          w = exp2f(ml.x - M);
          lpart += ml.y * w;
        }
      }
      s_w[tid] = w;
      __syncthreads();
      const int n = min(kCombineThreads, n_chunks - c0);
      const float* src = o_part + (base + (int64_t)c0 * H) * kLatent + c4;
      const int64_t step = (int64_t)H * kLatent;
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4*>(src + (j + u) * step);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += v[u] * s_w[j + u];
      }
      for (; j < n; ++j) acc += *reinterpret_cast<const f32x4*>(src + j * step) * s_w[j];
      __syncthreads();
    }
  }
  float Lsum = block_sum_128(lpart, red);
  if (lse_prev && mp != neg_inf) {
    const float w = exp2f(mp - M);
    Lsum += w;
    acc += *reinterpret_cast<const f32x4*>(o_prev + orow * kLatent + c4) * w;
  }
  const f32x4 res = Lsum > 0.f ? acc * (1.f / Lsum) : f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();                 // o_out / lse_out may alias o_prev / lse_prev
  *reinterpret_cast<f32x4*>(o_out + orow * kLatent + c4) = res;
  if (lse_out && tid == 0) lse_out[orow] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : neg_inf;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Plan {
  int n_sparse_tiles, n_window_tiles;
  int sparse_per_chunk, window_per_chunk, n_chunks;
};

static int head_groups(int32_t H) { return H % 32 == 0 ? H / 32 : H / 16; }

constexpr int kTargetWorkgroups = 512;         // two four-wave workgroups per CU
constexpr int kMinChunkTiles = 4;              // partial outputs stay small next to the gathered rows

// Chunks per (layer, row): about kTargetWorkgroups workgroups in total, at least
// kMinChunkTiles sparse tiles per chunk; the window tiles are spread one per
// chunk where there are enough chunks.
static Plan chunk_plan(int32_t L, int32_t R, int32_t H, int32_t K, bool sparse, bool window) {
  Plan p;
  p.n_sparse_tiles = sparse ? (K + kKT - 1) / kKT : 0;
  p.n_window_tiles = window ? kWindowChunks : 0;
  if (p.n_sparse_tiles == 0) {
    p.sparse_per_chunk = 0;
    p.n_chunks = p.n_window_tiles;
    p.window_per_chunk = 1;
    return p;
  }
  const int64_t per_chunk = (int64_t)L * R * head_groups(H);
  const int64_t want = (kTargetWorkgroups + per_chunk - 1) / per_chunk;
  int64_t spc = (p.n_sparse_tiles + want - 1) / want;
  if (spc < kMinChunkTiles) spc = kMinChunkTiles;
  if (spc > kMaxChunkTiles) spc = kMaxChunkTiles;
  if (spc > p.n_sparse_tiles) spc = p.n_sparse_tiles;
  p.sparse_per_chunk = (int)spc;
  p.n_chunks = (int)((p.n_sparse_tiles + spc - 1) / spc);
  p.window_per_chunk = p.n_window_tiles ? (p.n_window_tiles + p.n_chunks - 1) / p.n_chunks : 0;
  return p;
}

static size_t partial_bytes(int32_t L, int32_t R, int32_t H, int n_chunks, size_t* off_ml) {
  const size_t rows = (size_t)L * R * n_chunks * H;
  size_t o = align_up(rows * kLatent * sizeof(float), 256);
  size_t ml = align_up(rows * 2 * sizeof(float), 256);
  if (off_ml) *off_ml = o;
  return o + ml;
}

static bool heads_ok(int32_t H) { return H == 16 || H == 32 || H == 48 || H == 64; }

// Heads are split into groups of 32 (or 16 when H is not a multiple of 32),
// one workgroup per group: the 32-head kernel fits two waves per SIMD and two
// workgroups per CU, which hides barrier and memory latency better than one
// 64-head workgroup; the price is dequantising each tile once per group.
static void launch_chunks(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_chunks, a.R, a.head_groups * a.L);
  if (a.H % 32 == 0) attn_chunk_kernel<2><<<grid, 256, 0, s>>>(a);
  else attn_chunk_kernel<1><<<grid, 256, 0, s>>>(a);
}

// shared launch of L layers of one attention form (sparse part, window part or both);
// idx_off[l] is the element offset of layer l's index slice
static csa2_status attention_call(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* codes,
                                  const uint8_t* scales, int32_t B, int64_t T, const int32_t* row_seq,
                                  const int32_t* idx, const int64_t* idx_off, int32_t K, const uint16_t* swa,
                                  int32_t S, const int32_t* swa_start, const int32_t* swa_len, float softmax_scale,
                                  const float* o_prev, const float* lse_prev, float* o, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const PageMap& pm = PageMap{}) {
  const Plan p = chunk_plan(L, R, H, K, idx != nullptr, swa != nullptr);
  AttnArgs a;
  a.pm = pm;
  a.q_lat = q_lat; a.R = R; a.H = H; a.L = L; a.head_groups = head_groups(H);
  a.codes = codes; a.scales = scales; a.T = T; a.row_seq = row_seq;
  a.idx = idx; a.K = K;
  for (int l = 0; l < kMaxLayers; ++l) a.idx_off[l] = (idx && l < L) ? idx_off[l] : 0;
  a.n_sparse_tiles = p.n_sparse_tiles; a.n_window_tiles = p.n_window_tiles;
  a.window_per_chunk = p.window_per_chunk; a.sparse_per_chunk = p.sparse_per_chunk; a.n_chunks = p.n_chunks;
  a.swa = swa; a.B = B; a.S = S; a.swa_start = swa_start; a.swa_len = swa_len;
  a.scale_log2 = softmax_scale * kLog2e;
  size_t off_ml;
  const size_t need = partial_bytes(L, R, H, a.n_chunks, &off_ml);
  if (!workspace || workspace_bytes < need) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  a.o_part = static_cast<float*>(workspace);
  a.ml_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + off_ml);
  // one chunk per row and no prior result (many rows): the chunk kernel writes o and lse itself
  const bool direct = a.n_chunks == 1 && o_prev == nullptr && lse_prev == nullptr;
  a.o_out = direct ? o : nullptr;
  a.lse_out = direct ? lse : nullptr;
  hipStream_t s = (hipStream_t)stream;
  launch_chunks(a, s);
  if (!direct)
    attn_combine_kernel<<<dim3(H, R, L), kCombineThreads, 0, s>>>(a.o_part, a.ml_part, a.n_chunks, R, H, o_prev,
                                                                  lse_prev, o, lse);
  return launch_status();
}

static size_t attention_workspace(int32_t L, int32_t R, int32_t H, int32_t K, bool sparse, bool window) {
  return partial_bytes(L, R, H, chunk_plan(L, R, H, K, sparse, window).n_chunks, nullptr);
}

}  // namespace csa2

using namespace csa2;

static const int64_t kNoOffset[1] = {0};

extern "C" size_t csa2_sparse_decode_workspace_size(int32_t R, int32_t H, int32_t K) {
  if (R <= 0 || H <= 0 || K <= 0) return 0;
  return attention_workspace(1, R, H, K, true, false);
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
  return attention_call(1, q_lat, R, H, codes, scales, B, T, row_seq, idx, kNoOffset, K, nullptr, 0, nullptr,
                        nullptr, softmax_scale, nullptr, nullptr, o, lse, workspace, workspace_bytes, stream);
}

extern "C" size_t csa2_swa_merge_workspace_size(int32_t R, int32_t H) {
  if (R <= 0 || H <= 0) return 0;
  return attention_workspace(1, R, H, 0, false, true);
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
  return attention_call(1, q_lat, R, H, nullptr, nullptr, B, 0, row_seq, nullptr, nullptr, 0, swa, S, swa_start,
                        swa_len, softmax_scale, o_sparse, lse_sparse, o_out, lse_out, workspace, workspace_bytes,
                        stream);
}

extern "C" size_t csa2_sparse_swa_decode_workspace_size(int32_t R, int32_t H, int32_t K) {
  if (R <= 0 || H <= 0 || K <= 0) return 0;
  return attention_workspace(1, R, H, K, true, true);
}

static csa2_status check_sparse_swa(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* codes,
                                    const uint8_t* scales, int32_t B, int64_t T, const int32_t* row_seq,
                                    const int32_t* idx, int32_t K, const uint16_t* swa, int32_t S,
                                    const int32_t* swa_start, const int32_t* swa_len, const float* o,
                                    const float* lse) {
  if (!q_lat || !codes || !scales || !idx || !swa || !swa_start || !swa_len || !o || !lse) return CSA2_EINVAL;
  if (L <= 0 || R <= 0 || B <= 0 || T <= 0 || K <= 0 || S <= 0) return CSA2_EINVAL;
  if (L > kMaxLayers) return CSA2_ESHAPE;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (!heads_ok(H)) return CSA2_ESHAPE;
  if (T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_lat, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(idx, 4) || !aligned(swa, 16) ||
      !aligned(o, 16) || !aligned(lse, 4))
    return CSA2_EALIGN;
  return CSA2_OK;
}

extern "C" csa2_status csa2_sparse_swa_decode(const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* codes,
                                              const uint8_t* scales, int32_t B, int64_t T, const int32_t* row_seq,
                                              const int32_t* idx, int32_t K, const uint16_t* swa, int32_t S,
                                              const int32_t* swa_start, const int32_t* swa_len,
                                              float softmax_scale, float* o, float* lse, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  const csa2_status st = check_sparse_swa(1, q_lat, R, H, codes, scales, B, T, row_seq, idx, K, swa, S, swa_start,
                                          swa_len, o, lse);
  if (st != CSA2_OK) return st;
  return attention_call(1, q_lat, R, H, codes, scales, B, T, row_seq, idx, kNoOffset, K, swa, S, swa_start, swa_len,
                        softmax_scale, nullptr, nullptr, o, lse, workspace, workspace_bytes, stream);
}

extern "C" size_t csa2_sparse_swa_decode_layers_workspace_size(int32_t L, int32_t R, int32_t H, int32_t K) {
  if (L <= 0 || L > kMaxLayers || R <= 0 || H <= 0 || K <= 0) return 0;
  return attention_workspace(L, R, H, K, true, true);
}

extern "C" csa2_status csa2_sparse_swa_decode_layers(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H,
                                                     const uint8_t* codes, const uint8_t* scales, int32_t B,
                                                     int64_t T, const int32_t* row_seq, const int32_t* idx,
                                                     const int32_t* layer_idx, int32_t K, const uint16_t* swa,
                                                     int32_t S, const int32_t* swa_start, const int32_t* swa_len,
                                                     float softmax_scale, float* o, float* lse, void* workspace,
                                                     size_t workspace_bytes, void* stream) {
  const csa2_status st = check_sparse_swa(L, q_lat, R, H, codes, scales, B, T, row_seq, idx, K, swa, S, swa_start,
                                          swa_len, o, lse);
  if (st != CSA2_OK) return st;
  if (!layer_idx) return CSA2_EINVAL;
  int64_t off[kMaxLayers];
  for (int l = 0; l < L; ++l) {
    if (layer_idx[l] < 0) return CSA2_EINVAL;
    off[l] = (int64_t)layer_idx[l] * R * K;
  }
  return attention_call(L, q_lat, R, H, codes, scales, B, T, row_seq, idx, off, K, swa, S, swa_start, swa_len,
                        softmax_scale, nullptr, nullptr, o, lse, workspace, workspace_bytes, stream);
}

extern "C" csa2_status csa2_sparse_swa_decode_layers_paged(
    int32_t L, const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* code_pages, const uint8_t* scale_pages,
    int32_t B, int64_t T, const int32_t* row_seq, const int32_t* block_table, int64_t max_blocks, int32_t page,
    const int32_t* idx, const int32_t* layer_idx, int32_t K, const uint16_t* swa, int32_t S, const int32_t* swa_start,
    const int32_t* swa_len, float softmax_scale, float* o, float* lse, void* workspace, size_t workspace_bytes,
    void* stream) {
  csa2_status st = check_sparse_swa(L, q_lat, R, H, code_pages, scale_pages, B, T, row_seq, idx, K, swa, S,
                                    swa_start, swa_len, o, lse);
  if (st != CSA2_OK) return st;
  st = check_pages(block_table, max_blocks, page, T);
  if (st != CSA2_OK) return st;
  if (!layer_idx) return CSA2_EINVAL;
  int64_t off[kMaxLayers];
  for (int l = 0; l < L; ++l) {
    if (layer_idx[l] < 0) return CSA2_EINVAL;
    off[l] = (int64_t)layer_idx[l] * R * K;
  }
  return attention_call(L, q_lat, R, H, code_pages, scale_pages, B, T, row_seq, idx, off, K, swa, S, swa_start,
                        swa_len, softmax_scale, nullptr, nullptr, o, lse, workspace, workspace_bytes, stream,
                        PageMap{block_table, max_blocks, page});
}
