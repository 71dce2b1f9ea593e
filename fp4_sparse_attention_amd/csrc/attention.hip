// Sparse attention over the FP4 cache and sliding-window attention with
// log-sum-exp merge (HN summary key points: local sliding window plus global
// sparse retrieval over the shared main KV; MarkTechPost retelling, paragraph
// 2: a 128-token window in every layer).
//
// Absorbed multi-head latent attention: every head of a row attends over the
// same 512-channel latent rows, used as key and as value.
//
// Work split (split-K): a workgroup of four waves owns one query row of one
// layer and one chunk of its keys (a run of 32-key tiles from idx, plus up to
// one 32-row tile of the row's window), for all H <= 64 heads, so that every
// gathered tile is dequantised once for all heads.  Wave w owns latent
// channels [128 w, 128 w + 128).  Per tile:
//   A. the FP4 codes + scales of the tile's keys, gathered two tiles ahead into
//      registers, are dequantised in registers (v_cvt_scalef32_pk_f16_fp4 with
//      unit scale -- the instruction's scale acts only as a power of two --
//      times the E4M3 block scale in f16; exact, <= 6 significant bits in
//      [2^-10, 2688]) into the A operands of v_mfma_f32_32x32x16_f16; the wave
//      forms the partial scores S^T[key][head] over its 128 channels and leaves
//      its slice X[key][channel] in LDS;
//   B. the four partials meet in LDS; waves 0..H/16-1 sum them for 16 heads each
//      and run the softmax in the exp2 domain (one head per lane column),
//      publishing P (f16) in LDS; the head's running sum stays split over its
//      four lanes until the chunk ends;
//   C. O^T[channel][head] += X^T P^T for the wave's channels, X^T read from its
//      LDS slice with gfx950's transposing read (ds_read_b64_tr_b16), fp32
//      accumulators in registers.
// Two barriers per tile: the first region holds C of tile i - 1 and A of tile i,
// the second B of tile i, so the products of one tile overlap the
// dequantisation of the next.  The first two sparse tiles' rows are gathered
// with the query loads, with no barrier before the first tile, so that the
// gathers' latency overlaps the query loads; the window tile comes last.
//
// Exactness for every finite bf16 input: each wave's slice of each head's
// query is scaled by a power of two that puts the slice's largest magnitude at
// 2^15..2^16 before the f16 conversion (exact down to 2^-32 of that maximum),
// and the softmax multiplies the wave's partial score by the same power of two
// (exact) before the four are added; window rows, which are bf16 of any range,
// go through v_mfma_f32_32x32x16_bf16 for Q K^T (the same f16 query operands
// widened to bf16, exact) and, with P split into a bf16 high part and a bf16
// remainder, for P V.  Within a chunk there is no
// rescaling: P = 2^(s - m_ref) with m_ref set 8 above the first visible tile's
// maximum; a chunk whose scores pass m_ref + 15 (P would leave f16's range)
// restarts with m_ref = the largest score seen.
//
// The chunk's unnormalised O, running max m and sum l go to the workspace; a
// combine kernel merges the chunks (and, for a window merge, the sparse
// result) into o and lse.  When a row has one chunk and no prior result (enough
// rows to fill the chip, e.g. chunked prefill), the chunk kernel normalises and
// writes o and lse itself, with the combine's arithmetic for one chunk.
#include <type_traits>

#include "internal.hpp"

namespace csa2 {

constexpr int kKT = 32;                  // keys per tile
constexpr int kSStride = 36;             // floats per head row of a partial-score tile
constexpr int kPStride = 40;             // halfs per head row of P
constexpr int kXStride = 144;            // halfs per key row of a wave's dequantised tile slice (128 + 16 pad)
constexpr int kMaxChunkTiles = 64;       // sparse tiles per chunk at most
constexpr int kMaxChunkKeys = kMaxChunkTiles * kKT;
constexpr int kWindowChunks = kWindowMax / kKT;   // one-tile chunks covering the longest window
constexpr float kMaxSlack = 15.0f;       // P = 2^(s - m_ref) stays below 2^15 (f16 holds it)
constexpr float kRefLead = 8.0f;         // the reference starts this far above the first visible tile's max
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPrefetch = 2;             // sparse tiles whose gathers are in flight ahead of the math (4 ran 1.5-2 us
                                         // slower per 4-layer call: its registers cost the tile loop more than the cover gained)
constexpr int kMaxLayers = 8;
constexpr int kQTop = 15;                // a head's largest |q| is scaled to [2^15, 2^16)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16bf(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ s16x4 lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
}

// largest biased exponent field among 8 bf16 values (one uint4)
__device__ __forceinline__ uint32_t bf16x8_max_exp(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t e = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) e = max(e, max((w[i] >> 7) & 0xFFu, (w[i] >> 23) & 0xFFu));
  return e;
}

// 8 bf16 values times 2^-sh into f16 (exact for magnitudes >= 2^-17 after scaling)
__device__ __forceinline__ f16x8 bf16x8_scaled(uint4 v, int sh) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = (_Float16)__builtin_ldexpf(__uint_as_float(w[i] << 16), -sh);
    h[2 * i + 1] = (_Float16)__builtin_ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), -sh);
  }
  return h;
}

// 8 bf16 values times 2^-sh, as bf16 (exact unless the result leaves the fp32 range)
__device__ __forceinline__ bf16x8 bf16x8_scaled_bf16(uint4 v, int sh) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[2 * i] = (__bf16)__builtin_ldexpf(__uint_as_float(w[i] << 16), -sh);
    b[2 * i + 1] = (__bf16)__builtin_ldexpf(__uint_as_float(w[i] & 0xFFFF0000u), -sh);
  }
  return b;
}

// One launch covers L layers.  Layer l has its own queries, window rows and
// outputs, and reads the index slice at idx + idx_off[l] (layers may share one).
// Each (layer, row) splits its keys into n_chunks chunks: chunk c takes the
// window tiles [c wpc, (c+1) wpc) (tile w: rows [32w, 32w+32) of the window)
// and the sparse tiles [c spc, (c+1) spc).
struct AttnArgs {
  const uint16_t* q_lat;          // bf16 [L][R][H][512]
  int R, H, L;
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
  int n_wg;                       // L * R * n_chunks workgroups with work
  int per_xcd;                    // ceil(n_wg / 8): the slice of the (row, layer, chunk) list each XCD takes
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

// raw FP4 data of the lane's key for one tile (gathered kPrefetch tiles ahead):
// lane (key n, half h) of wave w holds codes of channels 128 w + 64 h + [0, 64)
// and the dword of their four block scales
struct RawTile {
  uint4 c0, c1;       // 32 code bytes
  uint32_t sc;        // 4 scale bytes
};

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32bf(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Workgroup id -> (row, layer, chunk): the eight XCDs take workgroup ids in
// turn (id b runs on XCD b mod 8), and XCD x takes the x-th contiguous slice of
// the list of (row, layer, chunk) triples, row-major, so that the chunks of one
// row -- which read the same queries, and for layers that share an index slice
// the same cache rows -- meet in one L2.
//
// Matrix-core layouts (v_mfma_f32_32x32x16_*, the full-rate shape on gfx950;
// the 16x16x32 shape issues at about half its rate), wave w, lane l with
// n = l % 32, h = l / 32:
//   operands: lane l holds row (or column) n, k = 8 h + j, j < 8; output:
//   lane l holds column n, rows 8 q + 4 h + r in register 4 q + r.
//   QK:  S^T[key][head] = X[key][ch] Q^T[ch][head]; k-step ks maps k = 8 h + j
//        to channel 128 w + 64 h + 8 ks + j (for X, lane n is key n; for Q^T
//        it is head 32 hb + n).  The output gives lane (n, h) keys 8 q + 4 h + r
//        of head 32 hb + n.  The lane also writes its 64 channels of key n to
//        the wave's slice X[key][channel] in LDS.
//   PV:  O^T[ch][head] += X^T P^T over channel blocks b (32 channels) and key
//        steps kk (16 keys): lane (n, h) supplies channel 32 b + n and keys
//        16 kk + 8 h + j of X^T (two transposing LDS reads), and for P^T the
//        same keys of head 32 hb + n, which the softmax lane (head, g = 2 kk +
//        h) writes as one 16-byte row.  Output lane (n, h) register 4 q + r is
//        head 32 hb + n, channel 128 w + 32 b + 8 q + 4 h + r.
template <int HB>
__global__ void __launch_bounds__(256, 1)
attn_chunk_kernel(const AttnArgs a) {
  constexpr int NH = 32 * HB;                 // heads, padded to whole 32-head blocks
  constexpr int NS = NH / 16;                 // softmax waves (16 heads each)
  __shared__ __attribute__((aligned(16))) float sp[4][NH * kSStride];
  __shared__ __attribute__((aligned(16))) uint16_t pp[2][NH * kPStride];
  __shared__ float s_inv_l[NH];
  __shared__ int s_restart;                   // a head's scores passed its reference by kMaxSlack
  __shared__ __attribute__((aligned(16))) float s_mask[kKT];
  __shared__ __attribute__((aligned(16))) int s_qsh[NH][4];      // query shift of (head, wave)
  __shared__ int s_pos[kMaxChunkKeys];        // this chunk's cache rows (-1: skip)
  __shared__ __attribute__((aligned(16))) uint16_t s_x[4][kKT * kXStride];   // each wave's tile slice X[key][ch]

  const int wg = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
  if (wg >= a.n_wg) return;
  const int chunk = wg % a.n_chunks;
  const int layer = (wg / a.n_chunks) % a.L;
  const int r = wg / (a.n_chunks * a.L);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;                    // matrix-core row / column
  const int hl = lane >> 5;                   // k half
  const int m = lane & 15;                    // softmax: head within the wave's 16
  const int g = lane >> 4;                    // softmax: key group 2 kk + h
  const int H = a.H;
  const int seq = a.row_seq ? a.row_seq[r] : r;
  const int cbase = 128 * wave;               // this wave's channel slice
  const float neg_inf = -__builtin_inff();

  // this chunk's tiles: sparse tiles [sp0, sp0 + n_sp), then window tiles [w0, w0 + n_wt)
  const int w0 = chunk * a.window_per_chunk;
  const int n_wt = max(0, min(a.n_window_tiles, w0 + a.window_per_chunk) - w0);
  const int sp0 = chunk * a.sparse_per_chunk;
  const int n_sp_real = max(0, min(a.n_sparse_tiles, sp0 + a.sparse_per_chunk) - sp0);
  // sparse tiles run in groups of kPrefetch, the last group padded with key-less
  // tiles, so that every step of the loop issues the same loads
  const int n_sp = (n_sp_real + kPrefetch - 1) / kPrefetch * kPrefetch;
  const int k0 = sp0 * kKT;
  const int k1 = min(a.K, (sp0 + n_sp_real) * kKT);

  // ---- loads, in the order they are issued: the index entries (this lane's key
  //      of each tile of the first group, and the chunk's entries for s_pos),
  //      the queries, the first window tile's rows, then -- once the first
  //      group's entries are in -- that group's cache rows, so that the gathers'
  //      latency overlaps the query loads (no barrier before the first tile)
  const int32_t* idx_row = n_sp > 0 ? a.idx + a.idx_off[layer] + (int64_t)r * a.K : nullptr;
  constexpr int kPosPerThread = kMaxChunkKeys / 256;
  int first_pos[kPrefetch];
  int chunk_pos[kPosPerThread];
  // (loads are unconditional, at clamped in-bounds addresses, and masked after
  // they return, so that no branch or wait sits between them)
  if (n_sp > 0) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) first_pos[j] = idx_row[min(k0 + j * kKT + n, k1 - 1)];
#pragma unroll
    for (int u = 0; u < kPosPerThread; ++u)
      if (256 * u < n_sp * kKT) chunk_pos[u] = idx_row[min(k0 + tid + 256 * u, k1 - 1)];
  }

  // queries (raw bf16): lane (n, h) holds channels cbase + 64 h + [0, 64) of head
  // 32 hb + n (zero past H)
  const uint16_t* q_l = a.q_lat + (int64_t)layer * a.R * H * kLatent;
  uint4 qraw[HB][8];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 32 * hb + n;
    const uint16_t* qrow = q_l + ((int64_t)r * H + min(head, H - 1)) * kLatent + cbase + 64 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qraw[hb][ks] = *reinterpret_cast<const uint4*>(qrow + 8 * ks);
  }

  // window rows of tile w: lane (n, h) takes channels cbase + 64 h + [0, 64) of
  // row 32 w + n; rows past the window's length read an in-bounds row (the loads
  // are unconditional) and are zeroed where they are used
  uint4 wv[8];
  bool wvalid = false;
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
    const int kk = w * kKT + n;
    wvalid = kk < w_ln;
    const uint4* p = reinterpret_cast<const uint4*>(swa_l + ((int64_t)seq * a.S + (wvalid ? w_st + kk : 0)) * kLatent +
                                                    cbase + 64 * hl);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) wv[ks] = p[ks];
  };
  if (n_wt > 0 && n_sp == 0) load_window(w0);

  // cache row of an index entry (page translation included; -1: skip); a row
  // of the codes array is below 2^31 (2^31 rows would be 618 GB)
  auto cache_row = [&](int pos) -> int {
    return (pos >= 0 && pos < a.T) ? (int)phys_row(a.pm, seq, a.T, pos) : -1;
  };
  // gather the FP4 codes + scales of one key into a register buffer (every load
  // is issued, an invalid key reading an in-bounds row, so the count of loads in
  // flight is the same on every path)
  auto load_row = [&](RawTile& raw, int row) {
    const int64_t rr = row >= 0 ? row : 0;
    const uint4* cp = reinterpret_cast<const uint4*>(a.codes + rr * kCodesRow + 64 * wave + 32 * hl);
    raw.c0 = cp[0];
    raw.c1 = cp[1];
    raw.sc = *reinterpret_cast<const uint32_t*>(a.scales + rr * kScalesRow + 8 * wave + 4 * hl);
  };
  // sparse tile j's key for this lane, from the staged rows
  auto load_tile = [&](RawTile& raw, int j) { load_row(raw, s_pos[j * kKT + n]); };
  RawTile buf[kPrefetch];
  if (n_sp > 0) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) load_row(buf[j], cache_row(k0 + j * kKT + n < k1 ? first_pos[j] : -1));
    // the chunk's cache rows, staged once so that the later gathers do not wait
    // on dependent index or page-table loads (visible after the barrier before
    // the sparse tiles)
#pragma unroll
    for (int u = 0; u < kPosPerThread; ++u) {
      const int i = tid + 256 * u;
      if (i < n_sp * kKT) s_pos[i] = cache_row(k0 + i < k1 ? chunk_pos[u] : -1);
    }
  }
  if (tid == 0) s_restart = 0;

  // ---- query shift of (head, wave): the largest exponent field over the wave's
  //      128 channels of the head puts that slice's largest magnitude at
  //      2^kQTop..2^(kQTop+1) in f16 (exact down to 2^-32 of it); the softmax
  //      multiplies each wave's partial score by 2^shift before adding them.
  //      Queries into f16 operands (window tiles widen them to bf16, exact).
  f16x8 qb[HB][8];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    // a padding head (32 hb + n >= H) read head H - 1's row: zero it
    if (32 * hb + n >= H) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qraw[hb][ks] = make_uint4(0, 0, 0, 0);
    }
    uint32_t e = 0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) e = max(e, bf16x8_max_exp(qraw[hb][ks]));
    auto sw32 = __builtin_amdgcn_permlane32_swap(e, e, false, false);
    e = max(sw32[0], sw32[1]);
    const int sh = (e == 0 ? -126 : (int)e - 127) - kQTop;
    if (hl == 0) s_qsh[32 * hb + n][wave] = sh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[hb][ks] = bf16x8_scaled(qraw[hb][ks], sh);
  }

  f32x16 oacc[4][HB];           // channel block b, head block hb
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) oacc[b][hb] = zero16();
  // per softmax lane: the head's reference max (fixed by its first visible tile,
  // or after a restart by every score seen), the largest score this lane saw, and
  // this lane's part of the sum
  float m_ref = neg_inf, m_seen = neg_inf;
  float l_run = 0.f;
  float fw[4] = {0.f, 0.f, 0.f, 0.f};
  bool fw_ready = false;

  // ---- A: partial scores of the tile into sp, and the wave's slice of the tile
  //      X[key][channel] (f16 for cache tiles, bf16 bits for window tiles) into
  //      s_x[wave] for the PV products, which read it transposed
  auto store_partials = [&](const f32x16 (&sacc)[HB]) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(&sp[wave][(32 * hb + n) * kSStride + 8 * q + 4 * hl]) =
            f32x4{sacc[hb][4 * q], sacc[hb][4 * q + 1], sacc[hb][4 * q + 2], sacc[hb][4 * q + 3]};
  };
  uint16_t* xrow = &s_x[wave][n * kXStride + 64 * hl];     // key n, this lane's 64 channels
  auto stage_sparse = [&](RawTile& raw, int j, bool refill) {
    const bool ok = s_pos[j * kKT + n] >= 0;
    // an invalid key gets scale 0 (its codes then dequantise to +-0) and a
    // masked score
    const uint32_t sc = ok ? raw.sc : 0u;
    const float sv[4] = {__builtin_amdgcn_cvt_f32_fp8((int)sc, 0), __builtin_amdgcn_cvt_f32_fp8((int)sc, 1),
                         __builtin_amdgcn_cvt_f32_fp8((int)sc, 2), __builtin_amdgcn_cvt_f32_fp8((int)sc, 3)};
    f16x2 hs[4];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) hs[bk] = f16x2{(_Float16)sv[bk], (_Float16)sv[bk]};
    const uint32_t cw[8] = {raw.c0.x, raw.c0.y, raw.c0.z, raw.c0.w, raw.c1.x, raw.c1.y, raw.c1.z, raw.c1.w};
    f32x16 sacc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) sacc[hb] = zero16();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f16x8 xa0 = fp4x8_to_f16(cw[2 * b], hs[b]);
      const f16x8 xa1 = fp4x8_to_f16(cw[2 * b + 1], hs[b]);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        sacc[hb] = mfma32(xa0, qb[hb][2 * b], sacc[hb]);
        sacc[hb] = mfma32(xa1, qb[hb][2 * b + 1], sacc[hb]);
      }
      *reinterpret_cast<f16x8*>(xrow + 16 * b) = xa0;
      *reinterpret_cast<f16x8*>(xrow + 16 * b + 8) = xa1;
    }
    store_partials(sacc);
    if (wave == 0 && hl == 0) s_mask[n] = ok ? 0.f : neg_inf;
    // buffer free: refill it with the tile kPrefetch ahead (every group but the
    // last has one)
    if (refill) load_tile(raw, j + kPrefetch);
  };
  // f16 query operand widened to bf16 (exact: a scaled bf16 value in f16 keeps
  // its 8 significant bits)
  auto q_bf16 = [&](const f16x8& h) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (__bf16)(float)h[i];
    return o;
  };
  auto stage_window = [&]() {
    const uint4 zero = make_uint4(0, 0, 0, 0);
    f32x16 sacc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) sacc[hb] = zero16();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint4 w0 = wvalid ? wv[2 * b] : zero, w1 = wvalid ? wv[2 * b + 1] : zero;
      const bf16x8 xa0 = __builtin_bit_cast(bf16x8, w0);
      const bf16x8 xa1 = __builtin_bit_cast(bf16x8, w1);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        sacc[hb] = mfma32bf(xa0, q_bf16(qb[hb][2 * b]), sacc[hb]);
        sacc[hb] = mfma32bf(xa1, q_bf16(qb[hb][2 * b + 1]), sacc[hb]);
      }
      *reinterpret_cast<uint4*>(xrow + 16 * b) = w0;
      *reinterpret_cast<uint4*>(xrow + 16 * b + 8) = w1;
    }
    store_partials(sacc);
    if (wave == 0 && hl == 0) s_mask[n] = wvalid ? 0.f : neg_inf;
  };

  // ---- B: softmax of the tile for heads [16 w, 16 w + 16): lane (m, g) owns head
  //      16 w + m and keys 8 g .. 8 g + 7; P goes to LDS (f16, or for a window
  //      tile bf16 high parts and bf16 remainders)
  auto softmax = [&](bool win) {
    if (wave >= NS) return;
    const int head = 16 * wave + m;
    const int kb = 8 * g;
    // each wave's partial score times 2^(its query shift) (exact), summed in fp32;
    // the four factors are read once, at the first tile (past a barrier)
    if (!fw_ready) {
      const int4 shv = *reinterpret_cast<const int4*>(&s_qsh[head][0]);
      fw[0] = __builtin_ldexpf(1.f, shv.x);
      fw[1] = __builtin_ldexpf(1.f, shv.y);
      fw[2] = __builtin_ldexpf(1.f, shv.z);
      fw[3] = __builtin_ldexpf(1.f, shv.w);
      fw_ready = true;
    }
    float s[8];
    {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&sp[0][head * kSStride + kb]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&sp[0][head * kSStride + kb + 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) { s[q] = v0[q] * fw[0]; s[4 + q] = v1[q] * fw[0]; }
    }
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&sp[w2][head * kSStride + kb]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&sp[w2][head * kSStride + kb + 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[q] = __builtin_fmaf(v0[q], fw[w2], s[q]);
        s[4 + q] = __builtin_fmaf(v1[q], fw[w2], s[4 + q]);
      }
    }
    const f32x4 mk0 = *reinterpret_cast<const f32x4*>(&s_mask[kb]);
    const f32x4 mk1 = *reinterpret_cast<const f32x4*>(&s_mask[kb + 4]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[q] = __builtin_fmaf(s[q], a.scale_log2, mk0[q]);
      s[4 + q] = __builtin_fmaf(s[4 + q], a.scale_log2, mk1[q]);
    }
    // this lane's max; the head's four lanes (g) meet only where they must
    const float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    m_seen = fmaxf(m_seen, mx);
    // no rescaling of O inside the chunk: P = 2^(s - m_ref) with the reference
    // set kRefLead above the head's first visible tile's max (a cross-lane max,
    // taken only while some head of the wave has no reference yet); a score more
    // than kMaxSlack above the reference (P would pass 2^15) makes the workgroup
    // redo the chunk with the largest score seen as the reference
    if (__any(m_ref == neg_inf)) {
      const float hm = xor32_max(xor16_max(mx));
      if (m_ref == neg_inf && hm != neg_inf) m_ref = hm + kRefLead;
    }
    if (mx > m_ref + kMaxSlack) s_restart = 1;
    const float m_use = m_ref == neg_inf ? 0.f : m_ref;     // nothing visible yet: every p is 0
    float p[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      p[q] = __builtin_amdgcn_exp2f(s[q] - m_use);
      l_run += p[q];            // this lane's share of the sum (the head's lanes are added at the end)
    }
    if (!win) {
      f16x8 ph;
#pragma unroll
      for (int q = 0; q < 8; ++q) ph[q] = (_Float16)p[q];
      *reinterpret_cast<f16x8*>(&pp[0][head * kPStride + 8 * g]) = ph;
    } else {
      bf16x8 hi, lo;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        hi[q] = (__bf16)p[q];
        lo[q] = (__bf16)(p[q] - (float)hi[q]);
      }
      *reinterpret_cast<bf16x8*>(&pp[0][head * kPStride + 8 * g]) = hi;
      *reinterpret_cast<bf16x8*>(&pp[1][head * kPStride + 8 * g]) = lo;
    }
  };

  // ---- C: O^T[block b][head block hb] += X^T P^T for the tile in s_x[wave]
  //      (kind 0 f16 cache tile, 1 bf16 window tile) whose P is in LDS.  Lane
  //      (m, G) = (l % 16, l / 16) reads with ds_read_b64_tr_b16 the keys
  //      16 kk + 8 (G / 2) + j, j < 8, of channel 32 b + 16 (G % 2) + m: the A
  //      operand rows are the block's channels in order, k its keys in order
  const uint16_t* xtr = &s_x[wave][(8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * kXStride + 16 * ((lane >> 4) & 1) +
                                   4 * (lane & 3)];
  auto pv = [&](int kind) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 ph[HB], pl[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int prow = (32 * hb + n) * kPStride + 8 * (2 * kk + hl);
        ph[hb] = *reinterpret_cast<const uint4*>(&pp[0][prow]);
        if (kind == 1) pl[hb] = *reinterpret_cast<const uint4*>(&pp[1][prow]);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint16_t* p = xtr + 16 * kk * kXStride + 32 * b;
        const s16x4 lo = lds_tr16(p), hi = lds_tr16(p + 4 * kXStride);
        const short x8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          if (kind == 0) {
            oacc[b][hb] = mfma32(__builtin_bit_cast(f16x8, x8), __builtin_bit_cast(f16x8, ph[hb]), oacc[b][hb]);
          } else {
            const bf16x8 x = __builtin_bit_cast(bf16x8, x8);
            oacc[b][hb] = mfma32bf(x, __builtin_bit_cast(bf16x8, ph[hb]), oacc[b][hb]);
            oacc[b][hb] = mfma32bf(x, __builtin_bit_cast(bf16x8, pl[hb]), oacc[b][hb]);
          }
        }
      }
    }
  };

  // ---- the pipelined loop over the sparse tiles: step j holds C of tile j - 1
  //      (its slice still in LDS, its P in LDS) and A of tile j, then B of
  //      tile j; the last group is peeled so that it issues no refills.
  //      (Scheduling barriers keep each step's instructions in place.)
  auto sparse_step = [&](RawTile& raw, int j, bool refill) {
    __builtin_amdgcn_sched_barrier(0);
    if (j > 0) pv(0);           // the previous tile, whose slice s_x[wave] still holds
    stage_sparse(raw, j, refill);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    softmax(false);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  bool first_pass = true;
  for (;;) {
    if (n_sp > 0) {
      // (the first pass's first group was gathered in the prologue)
      if (!first_pass) {
#pragma unroll
        for (int b = 0; b < kPrefetch; ++b) load_tile(buf[b], b);
      }
      __syncthreads();          // the staged rows and the query shifts are visible
      for (int j = 0; j < n_sp - kPrefetch; j += kPrefetch) {
#pragma unroll
        for (int b = 0; b < kPrefetch; ++b) sparse_step(buf[b], j + b, true);
      }
      const int jl = n_sp - kPrefetch;
#pragma unroll
      for (int b = 0; b < kPrefetch; ++b) sparse_step(buf[b], jl + b, false);
      pv(0);
    }
    // ---- window tiles, after the sparse ones (bf16 products; not pipelined);
    //      a window-only chunk's first rows were loaded with the queries
    for (int i = 0; i < n_wt; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i > 0 || n_sp > 0 || !first_pass) load_window(w0 + i);
      __syncthreads();          // every wave is past the previous tile's P reads
      stage_window();
      __syncthreads();
      softmax(true);
      __syncthreads();
      pv(1);
    }
    __syncthreads();
    if (!s_restart) break;
    // restart: every head's reference becomes its largest score (P <= 1 from now on)
    __syncthreads();
    if (tid == 0) s_restart = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) oacc[b][hb] = zero16();
    m_ref = xor32_max(xor16_max(m_seen));
    l_run = 0.f;
    first_pass = false;
  }

  // the head's sum over its four softmax lanes
  l_run = xor32_sum(xor16_sum(l_run));

  // ---- outputs: lane (n, h) register 4 q + i of block (b, hb) is head 32 hb + n,
  //      channel cbase + 32 b + 8 q + 4 h + i
  const int64_t orow0 = ((int64_t)layer * a.R + r) * H;
  if (a.o_out) {
    // the row's only chunk and no prior: normalise here, as the combine would for one chunk
    if (wave < NS && g == 0) s_inv_l[16 * wave + m] = l_run > 0.f ? 1.f / l_run : 0.f;
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = 32 * hb + n;
      if (head >= H) continue;
      const float inv = s_inv_l[head];
      float* op = a.o_out + (orow0 + head) * kLatent + cbase + 4 * hl;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {oacc[b][hb][4 * q], oacc[b][hb][4 * q + 1], oacc[b][hb][4 * q + 2], oacc[b][hb][4 * q + 3]};
          *reinterpret_cast<f32x4*>(op + 32 * b + 8 * q) =
              inv > 0.f ? v * inv : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (a.lse_out && wave < NS && g == 0 && 16 * wave + m < H)
      a.lse_out[orow0 + 16 * wave + m] = l_run > 0.f ? (m_ref + log2f(l_run)) * kLn2 : neg_inf;
    return;
  }
  // ---- this chunk's partial: unnormalised O, and (m, l) from the softmax owners
  const int64_t prow0 = (((int64_t)layer * a.R + r) * a.n_chunks + chunk) * H;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 32 * hb + n;
    if (head >= H) continue;
    float* op = a.o_part + (prow0 + head) * kLatent + cbase + 4 * hl;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(op + 32 * b + 8 * q) =
            f32x4{oacc[b][hb][4 * q], oacc[b][hb][4 * q + 1], oacc[b][hb][4 * q + 2], oacc[b][hb][4 * q + 3]};
  }
  if (wave < NS && g == 0 && 16 * wave + m < H) {
    a.ml_part[(prow0 + 16 * wave + m) * 2 + 0] = m_ref;
    a.ml_part[(prow0 + 16 * wave + m) * 2 + 1] = l_run;
  }
}

// The combine's workgroup -> (layer, row, head): XCD x (workgroup ids b with
// b mod 8 = x) takes the (layer, row) pairs whose first chunk the chunk kernel
// ran on XCD x (about 1 us faster per 4-layer batch-8 call than the plain
// (head, row, layer) grid; the partials themselves still come from past the
// L2, which the kernel boundary writes back).  Pair p = row * L + layer owns chunk workgroups [p nc, p nc + nc) of
// the chunk kernel's list, of which XCD x took [x per_xcd, x per_xcd + per_xcd).
struct CombineMap {
  int L, R, H, n_chunks, per_xcd;
};

__device__ __forceinline__ int combine_pair_begin(const CombineMap& cm, int x) {
  const int64_t p = ((int64_t)x * cm.per_xcd + cm.n_chunks - 1) / cm.n_chunks;
  const int64_t P = (int64_t)cm.L * cm.R;
  return (int)(p < P ? p : P);
}

// false: a padding workgroup with no (layer, row, head)
__device__ __forceinline__ bool combine_item(const CombineMap& cm, int& h, int& r, int& layer) {
  const int x = (int)(blockIdx.x & 7), s = (int)(blockIdx.x >> 3);
  const int p0 = combine_pair_begin(cm, x);
  const int p1 = x == 7 ? cm.L * cm.R : combine_pair_begin(cm, x + 1);
  if (s >= (p1 - p0) * cm.H) return false;
  const int p = p0 + s / cm.H;
  h = s % cm.H;
  r = p / cm.L;
  layer = p % cm.L;
  return true;
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
attn_combine_kernel(const float* __restrict__ o_part, const float* __restrict__ ml_part, const CombineMap cm,
                    const float* __restrict__ o_prev, const float* __restrict__ lse_prev,
                    float* __restrict__ o_out, float* __restrict__ lse_out) {
  __shared__ float s_w[kCombineThreads];
  __shared__ float red[2];
  int h, r, layer;
  if (!combine_item(cm, h, r, layer)) return;
  const int n_chunks = cm.n_chunks, R = cm.R, H = cm.H;
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

// The same merge for rows of at most kCombineFew chunks (the decode shapes):
// every thread loads every chunk's (m, l) and its four channels of every
// partial at once, so the kernel waits for one round of loads, with no LDS or
// barriers; the arithmetic is the general kernel's, chunk by chunk in order.
constexpr int kCombineFew = 16;

__global__ void __launch_bounds__(kCombineThreads)
attn_combine_few_kernel(const float* __restrict__ o_part, const float* __restrict__ ml_part, const CombineMap cm,
                        const float* __restrict__ o_prev, const float* __restrict__ lse_prev,
                        float* __restrict__ o_out, float* __restrict__ lse_out) {
  int h, r, layer;
  if (!combine_item(cm, h, r, layer)) return;
  const int n_chunks = cm.n_chunks, R = cm.R, H = cm.H;
  const int c4 = threadIdx.x * 4;
  const int64_t base = (((int64_t)layer * R + r) * n_chunks) * H + h;       // + chunk * H
  const int64_t orow = ((int64_t)layer * R + r) * H + h;
  const float neg_inf = -__builtin_inff();
  float2 ml[kCombineFew];
  f32x4 v[kCombineFew];
#pragma unroll
  for (int c = 0; c < kCombineFew; ++c) {
    if (c < n_chunks) {
      ml[c] = *reinterpret_cast<const float2*>(ml_part + (base + (int64_t)c * H) * 2);
      v[c] = *reinterpret_cast<const f32x4*>(o_part + (base + (int64_t)c * H) * kLatent + c4);
    }
  }
  float M = neg_inf;
#pragma unroll
  for (int c = 0; c < kCombineFew; ++c)
    if (c < n_chunks && ml[c].y > 0.f) M = fmaxf(M, ml[c].x);
  float mp = neg_inf;
  if (lse_prev) {
    mp = lse_prev[orow] * kLog2e;
    M = fmaxf(M, mp);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float Lsum = 0.f;
  if (M != neg_inf) {
#pragma unroll
    for (int c = 0; c < kCombineFew; ++c)
      if (c < n_chunks && ml[c].y > 0.f) {
        const float w = exp2f(ml[c].x - M);
        Lsum += ml[c].y * w;
        acc += v[c] * w;
      }
  }
  if (lse_prev && mp != neg_inf) {
    const float w = exp2f(mp - M);
    Lsum += w;
    acc += *reinterpret_cast<const f32x4*>(o_prev + orow * kLatent + c4) * w;
  }
  const f32x4 res = Lsum > 0.f ? acc * (1.f / Lsum) : f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();                 // o_out / lse_out may alias o_prev / lse_prev
  *reinterpret_cast<f32x4*>(o_out + orow * kLatent + c4) = res;
  if (lse_out && threadIdx.x == 0) lse_out[orow] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : neg_inf;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Plan {
  int n_sparse_tiles, n_window_tiles;
  int sparse_per_chunk, window_per_chunk, n_chunks;
};

constexpr int kMinChunkTiles = 4;              // partial outputs stay small next to the gathered rows

// Chunks per (layer, row): about one workgroup per compute unit in total, whole
// groups of kPrefetch sparse tiles per chunk; the window tiles are spread one
// per chunk where there are enough chunks.
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
  const int64_t per_chunk = (int64_t)L * R;
  const int64_t target = device_cu_count();
  const int64_t want = (target + per_chunk - 1) / per_chunk;
  int64_t spc = (p.n_sparse_tiles + want - 1) / want;
  // a latency-bound call whose chunk partials stay small even at one prefetch group per chunk (within 256 KB
  // in all: a single row of a few heads) may use such chunks (one row of 16 heads, K = 256: 16.3 -> 12.5 us
  // per call; two rows of 64 heads at K = 2,048, 8 MB of partials that way, ran 0.4 us slower)
  const int64_t small_parts = (int64_t)((p.n_sparse_tiles + kPrefetch - 1) / kPrefetch) * L * R * H * kLatent * 4;
  const int64_t min_tiles = small_parts <= (256 << 10) ? kPrefetch : kMinChunkTiles;
  if (spc < min_tiles) spc = min_tiles;
  spc = (spc + kPrefetch - 1) / kPrefetch * kPrefetch;     // whole groups of tiles
  if (spc > kMaxChunkTiles) spc = kMaxChunkTiles;
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

// One workgroup per (row, layer, chunk) with every head; XCD x takes the x-th
// slice of per_xcd of them
static void launch_chunks(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(8 * a.per_xcd));
  if (a.H <= 32) attn_chunk_kernel<1><<<grid, 256, 0, s>>>(a);
  else attn_chunk_kernel<2><<<grid, 256, 0, s>>>(a);
}

// shared launch of L layers of one attention form (sparse part, window part or both);
// idx_off[l] is the element offset of layer l's index slice
static csa2_status attention_call(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* codes,
                                  const uint8_t* scales, int32_t B, int64_t T, const int32_t* row_seq,
                                  const int32_t* idx, const int64_t* idx_off, int32_t K, const uint16_t* swa,
                                  int32_t S, const int32_t* swa_start, const int32_t* swa_len, float softmax_scale,
                                  const float* o_prev, const float* lse_prev, float* o, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  const PageMap& pm = PageMap{}, bool scratch = false) {
  const Plan p = chunk_plan(L, R, H, K, idx != nullptr, swa != nullptr);
  AttnArgs a;
  a.pm = pm;
  a.q_lat = q_lat; a.R = R; a.H = H; a.L = L;
  a.codes = codes; a.scales = scales; a.T = T; a.row_seq = row_seq;
  a.idx = idx; a.K = K;
  for (int l = 0; l < kMaxLayers; ++l) a.idx_off[l] = (idx && l < L) ? idx_off[l] : 0;
  a.n_sparse_tiles = p.n_sparse_tiles; a.n_window_tiles = p.n_window_tiles;
  a.window_per_chunk = p.window_per_chunk; a.sparse_per_chunk = p.sparse_per_chunk; a.n_chunks = p.n_chunks;
  a.n_wg = L * R * p.n_chunks;
  a.per_xcd = (a.n_wg + 7) / 8;
  a.swa = swa; a.B = B; a.S = S; a.swa_start = swa_start; a.swa_len = swa_len;
  a.scale_log2 = softmax_scale * kLog2e;
  size_t off_ml;
  const size_t need = partial_bytes(L, R, H, a.n_chunks, &off_ml);
  // one chunk per row and no prior result (many rows): the chunk kernel writes o and lse itself
  const bool direct = a.n_chunks == 1 && o_prev == nullptr && lse_prev == nullptr;
  if (scratch) {
    // the fixed static array: only partials use it
    if (!direct && need > workspace_bytes) return CSA2_ESCRATCH;
  } else if (!workspace || workspace_bytes < need) {
    return CSA2_EWORKSPACE;
  }
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  a.o_part = static_cast<float*>(workspace);
  a.ml_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + off_ml);
  a.o_out = direct ? o : nullptr;
  a.lse_out = direct ? lse : nullptr;
  hipStream_t s = (hipStream_t)stream;
  {
    // the index slices the layers read: [0, (largest offset) + R K)
    int64_t n_idx = 0;
    for (int l = 0; idx && l < L; ++l) n_idx = std::max<int64_t>(n_idx, idx_off[l] + (int64_t)R * K);
    const csa2_status dc = debug_check(row_seq, R, B, swa ? swa_start : nullptr, swa ? swa_len : nullptr,
                                       (int64_t)L * R, S, idx, n_idx, T, s);
    if (dc != CSA2_OK) return dc;
  }
  launch_chunks(a, s);
  if (!direct) {
    const CombineMap cm{L, R, H, a.n_chunks, a.per_xcd};
    // the largest number of (layer, row) pairs one XCD combines (the same split as combine_pair_begin)
    const int64_t P = (int64_t)L * R;
    auto pair_begin = [&](int x) {
      const int64_t p = ((int64_t)x * a.per_xcd + a.n_chunks - 1) / a.n_chunks;
      return p < P ? p : P;
    };
    int64_t most = 0;
    for (int x = 0; x < 8; ++x) most = std::max<int64_t>(most, (x == 7 ? P : pair_begin(x + 1)) - pair_begin(x));
    const dim3 grid((unsigned)(8 * most * H));
    if (a.n_chunks <= kCombineFew)
      attn_combine_few_kernel<<<grid, kCombineThreads, 0, s>>>(a.o_part, a.ml_part, cm, o_prev, lse_prev, o, lse);
    else
      attn_combine_kernel<<<grid, kCombineThreads, 0, s>>>(a.o_part, a.ml_part, cm, o_prev, lse_prev, o, lse);
  }
  return launch_status();
}

static size_t attention_workspace(int32_t L, int32_t R, int32_t H, int32_t K, bool sparse, bool window) {
  return partial_bytes(L, R, H, chunk_plan(L, R, H, K, sparse, window).n_chunks, nullptr);
}

// The allocation-free call's chunk partials live in this array, one copy per
// GPU (the runtime places it when the code object loads on that GPU).  Host
// code never passes the name itself to a kernel: its device address, resolved
// once per device with that device current, is kept in scratch_dev[].
constexpr size_t kScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static std::atomic<void*> scratch_dev[kMaxDevices];

static void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_dev[dev].load(std::memory_order_acquire);
  if (p) return p;
  // two threads that race here both store the same address
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  scratch_dev[dev].store(p, std::memory_order_release);
  return p;
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

extern "C" csa2_status csa2_sparse_swa_decode_layers_noalloc(
    int32_t L, const uint16_t* q_lat, int32_t R, int32_t H, const uint8_t* codes, const uint8_t* scales, int32_t B,
    int64_t T, const int32_t* row_seq, const int32_t* idx, const int32_t* layer_idx, int32_t K, const uint16_t* swa,
    int32_t S, const int32_t* swa_start, const int32_t* swa_len, float softmax_scale, float* o, float* lse,
    void* stream) {
  const csa2_status st = check_sparse_swa(L, q_lat, R, H, codes, scales, B, T, row_seq, idx, K, swa, S, swa_start,
                                          swa_len, o, lse);
  if (st != CSA2_OK) return st;
  if (!layer_idx) return CSA2_EINVAL;
  int64_t off[kMaxLayers];
  for (int l = 0; l < L; ++l) {
    if (layer_idx[l] < 0) return CSA2_EINVAL;
    off[l] = (int64_t)layer_idx[l] * R * K;
  }
  // a shape beyond the array is refused before any HIP call
  const Plan p = chunk_plan(L, R, H, K, true, true);
  if (p.n_chunks > 1 && partial_bytes(L, R, H, p.n_chunks, nullptr) > kScratchBytes) return CSA2_ESCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return CSA2_ELAUNCH;
  return attention_call(L, q_lat, R, H, codes, scales, B, T, row_seq, idx, off, K, swa, S, swa_start, swa_len,
                        softmax_scale, nullptr, nullptr, o, lse, ws, kScratchBytes, stream, PageMap{}, true);
}
