// Indexer scoring kernels: Full mode (every visible position) and Reindex mode
// (only the candidate-pool positions), per the CSA2 roles paragraph of the
// MarkTechPost retelling of DeepSeek-V4.1-Flash.
//
// score(r, j) = sum_{d<64} q_idx[r][d] * k_idx[seq(r)][j][d] with E4M3 inputs.
// The E4M3 bytes are widened to f16 (exact, v_cvt_scalef32_pk_f16_fp8 with unit
// scale) and multiplied on the f16 matrix cores, v_mfma_f32_16x16x32_f16
// (C[16 x 16] += A[16 x 32] * B[32 x 16]), in the tile layout of tile.hpp: a
// tile is 32 keys, each 16-key half takes two k-steps of 32 channels, and A
// holds the query in row 0 (decode) or 16 query rows of one sequence (chunked
// prefill), so every kernel forms a score from the same two steps and all of
// them agree bit for bit.  The products are exact; the matrix core adds a
// step's 32 products and the accumulator, rounding to fp32.  For unit-normal
// E4M3 inputs the score is the exact value rounded once; over the whole E4M3
// range the error measured stays below 2^-21 * sum |q_d k_d|.  (The fp8 matrix
// path is not used: its internal accumulation keeps only ~20 bits below the
// largest product.)  Each of a lane's two 16-byte loads per tile lies in a 1 KB
// stretch of 16 whole keys that the wave reads together.
//
// Decode (one query per sequence) is HBM-bound: 64 bytes of key per score; the
// matrix cores and the conversions use a small share of their peak.  Chunked
// prefill fills all 32 rows of A and is bound by the fp32 score writes.
#include <algorithm>

#include "internal.hpp"
#include "tile.hpp"

namespace csa2 {

// One query row per workgroup row (grid.y = R).  Used for decode (Full and
// Reindex).  kGather: column c of row r scores position pool[r][c].  kFp8:
// scores through the FP8 matrix instruction (csa2_index_full_fp8).
template <bool kGather, bool kFp8 = false, bool kPaged = false>
__global__ void __launch_bounds__(256)
index_rows_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                  const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                  const int32_t* __restrict__ pool, int64_t n_cols, float* __restrict__ scores,
                  int tiles_per_block, PageMap pm) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kn = lane & 15;          // the lane's keys kn and kn + 16 of each tile
  const int part = 16 * (lane >> 4); // and its 16 bytes of them
  const int seq = row_seq ? row_seq[r] : r;
  const int64_t limit = row_limit ? row_limit[r] : T - 1;
  float* out = scores + (int64_t)r * n_cols;
  const int32_t* prow = kGather ? pool + (int64_t)r * n_cols : nullptr;

  f16x8 a[2];
  long a8[2];
  if constexpr (kFp8) query_operands_fp8(q_idx + (int64_t)r * kIndexDim, lane, a8);
  else query_operands(q_idx + (int64_t)r * kIndexDim, lane, a);

  const int64_t n_tiles = (n_cols + kTile - 1) / kTile;
  const int64_t t_begin = (int64_t)blockIdx.x * tiles_per_block;
  const int64_t t_end = min(n_tiles, t_begin + tiles_per_block);
  const float neg_inf = -__builtin_inff();

  for (int64_t t0 = t_begin + wave; t0 < t_end; t0 += 4 * kUnroll) {
    i32x8 b[kUnroll];
    bool ok[kUnroll][2];
    // every load unconditional, at a clamped index (column 0, key row 0) and masked after: a load under a
    // branch made the compiler wait for each pool id before issuing the next
    int64_t p[kUnroll][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t c = (t0 + 4 * u) * kTile + 16 * h + kn;
        const bool in = t0 + 4 * u < t_end && c < n_cols;
        if (kGather) {
          const int64_t pv = (int64_t)prow[in ? c : 0];
          p[u][h] = in ? pv : -1;
        } else {
          p[u][h] = in ? c : -1;
        }
      }
    uint4 v[kUnroll][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t q = p[u][h];
        const bool vis = q >= 0 && q < T && q <= limit;
        // the dense layout as plain arithmetic (a page-table branch here made every key load wait)
        const int64_t row = !vis ? -1 : (kPaged ? phys_row(pm, seq, T, q) : (int64_t)seq * T + q);
        ok[u][h] = row >= 0;
        v[u][h] = load_key_part(k_idx + (ok[u][h] ? row : 0) * kIndexDim + part);
      }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (!ok[u][h]) v[u][h] = make_uint4(0, 0, 0, 0);
      b[u] = tile_pair(v[u][0], v[u][1]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = t0 + 4 * u;
      const float2 sc = kFp8 ? mfma_score_fp8(a8, b[u]) : mfma_score(a, b[u]);
      const int64_t c = t * kTile + kn;
      if (t < t_end && lane < 16) {
        if (c < n_cols) out[c] = ok[u][0] ? sc.x : neg_inf;
        if (c + 16 < n_cols) out[c + 16] = ok[u][1] ? sc.y : neg_inf;
      }
    }
  }
}

// Full-mode decode scan as a persistent kernel over units of 16 tiles (512
// positions).  The grid holds as many workgroups as the chip keeps resident.
// The next unit's keys are loaded before the current unit's products, so every
// wave keeps 8 KB in flight.  Wave w of unit j scores tiles 16j + 4w + i,
// i < 4: the 128-position block 4j + w.  Two unit orders:
//  - scores only: units row-major over all rows, workgroup b takes units b,
//    b + G, b + 2G, ...; at any time the grid reads one contiguous stretch of
//    the keys (the fastest order measured).
//  - kCand: each workgroup stays within one row (with R <= G, workgroup b
//    serves row b % R and takes its units b / R, b / R + G / R, ...; with
//    R > G, whole rows b, b + G, ...).  Besides the scores, each wave stores
//    its block's candidates (visible keys >= tau_s) in position order at the
//    block's start as (key, position) pairs (ballot ranks, no atomics), with the
//    block's count; the workgroup counts the candidates' histogram digits in
//    LDS (atomics without return: a returning atomic per candidate tile stalled
//    the wave, 17 us of the 8 x 1M scan) and adds its nonzero bins to the row's
//    histogram when it leaves the row (once per workgroup; with row-major
//    order every workgroup would flush at each row boundary, measured slower).
constexpr int kUnitTiles = 16;

// Sampling for the candidate threshold (the sample and threshold kernels below)
constexpr int kSampleN = 4096;
constexpr int kSampleRun = 8;

// rank m of the sample key that bounds a selection of k among V visible positions (0: take every position)
__device__ __forceinline__ uint32_t sample_rank(int32_t k, int64_t V) {
  if (V <= 0) return 0u;
  const double mu = (double)k * (double)kSampleN / (double)V;
  const double m = ceil(mu + 4.0 * sqrt(mu) + 8.0);
  return m > (double)kSampleN ? 0u : (uint32_t)m;
}

// The threshold kernel's steps by the 256 threads of a scan workgroup, for
// row r's 4,096 sample keys (16 per thread, loaded by sample_load_256): tau_s,
// the lower edge of the 22-bit key prefix holding the m-th largest sample
// (digits of 12 and 10 bits), and sh from the sample maximum.  h: 4,096 LDS
// words, zero on entry and on return; wt: 8 words; res: 2 words.
constexpr int kSamplePer = kSampleN / 256;

// Issued before the workgroup's first key loads: loads complete in issue
// order, so sample keys loaded after them would wait for the whole unit.
__device__ __forceinline__ void sample_load_256(const uint32_t* __restrict__ samp_row, uint32_t (&key)[kSamplePer]) {
  const uint4* s4 = reinterpret_cast<const uint4*>(samp_row) + (kSamplePer / 4) * threadIdx.x;
#pragma unroll
  for (int q = 0; q < kSamplePer / 4; ++q) {
    const uint4 v = s4[q];
    key[4 * q] = v.x; key[4 * q + 1] = v.y; key[4 * q + 2] = v.z; key[4 * q + 3] = v.w;
  }
}

__device__ void sample_threshold_256(const uint32_t (&key)[kSamplePer], int64_t V, int32_t k, uint32_t* h,
                                     uint32_t* wt, uint32_t* res, uint32_t& tau_s, uint32_t& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t m = sample_rank(k, V);
  if (m == 0u) {
    tau_s = 0u;
    sh = 21u;             // (key >> 21) < 2048 for every key
    return;
  }
  constexpr int kPer = kSamplePer;
  uint32_t kmax = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    kmax = max(kmax, key[j]);
    atomicAdd(&h[key[j] >> 20], 1u);
  }
  __syncthreads();
  uint32_t need = m;
  find_bin_256<4096>(h, need, wt, res);
  __syncthreads();
  uint32_t prefix = res[0] << 20;
  need -= res[1];
#pragma unroll
  for (int j = 0; j < 16; ++j) h[16 * tid + j] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if ((key[j] >> 20) == (prefix >> 20)) atomicAdd(&h[(key[j] >> 10) & 1023u], 1u);
  __syncthreads();
  find_bin_256<1024>(h, need, wt, res);
  kmax = wave_max_u32(kmax);
  if (lane == 0) wt[4 + wave] = kmax;
  __syncthreads();
  prefix |= res[0] << 10;
  const uint32_t mx = max(max(wt[4], wt[5]), max(wt[6], wt[7]));
#pragma unroll
  for (int j = 0; j < 4; ++j) h[4 * tid + j] = 0u;
  __syncthreads();
  const uint32_t span = mx - prefix;      // mx >= prefix: prefix is at most a sample key
  const int bits = span ? 32 - __builtin_clz(span) : 0;
  tau_s = prefix;
  sh = (uint32_t)(bits > 11 ? bits - 11 : 0);
}

// kPaged: keys in a page pool (pm.table set); kOut: scores written (always
// for the scores-only scan).  Both are template switches so that the common
// decode scan carries no page translation and no score stores.
template <bool kCand, bool kPaged, bool kOut>
__global__ void __launch_bounds__(256)
index_stream_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                    float* __restrict__ scores, int R, int64_t units_per_row, CandOut cand, PageMap pm) {
  __shared__ uint32_t h[kCand ? kStreamBins : 1];
  __shared__ uint32_t s_wt[kCand ? 8 : 1], s_res[kCand ? 2 : 1];
  // each wave's candidates (with their slots in the row's block area) held back in LDS and written out in
  // bursts when the stage fills and when the workgroup leaves the row: stores mixed into the key stream, one
  // per ballot, had cost ~4.5 us of the 8 x 1M scan (a per-block burst did not help; a per-row one does)
  constexpr int kStage = 512;
  __shared__ uint2 s_ent[kCand ? 4 : 1][kCand ? kStage : 1];
  __shared__ uint32_t s_dst[kCand ? 4 : 1][kCand ? kStage : 1];
  uint32_t n_st = 0;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kn = lane & 15;          // the lane's keys kn and kn + 16 of each tile
  const int part = 16 * (lane >> 4); // and its 16 bytes of them
  const float neg_inf = -__builtin_inff();
  const int G = gridDim.x;
  const int b = blockIdx.x;

  // the unit order (r = row, j = unit within the row; r reaches R at the end)
  int r;
  int64_t j;
  int row_step = 0;
  int64_t j0 = 0, j_step = 0;
  if (!kCand) {
    // all units row-major, workgroup b takes units b, b + G, ...
    if ((int64_t)b >= (int64_t)R * units_per_row) return;
    r = (int)(b / units_per_row);
    j = b - (int64_t)r * units_per_row;
  } else if (R <= G) {
    // workgroup b serves row b % R, units b / R, b / R + G / R, ...
    r = b % R;
    row_step = R;
    j0 = b / R;
    j_step = G / R;
    if (j0 >= units_per_row) return;
    j = j0;
  } else {
    // workgroup b scores the whole rows b, b + G, ...
    r = b;
    row_step = G;
    j_step = 1;
    j = 0;
  }
  auto advance = [&](int& rr, int64_t& jj) {
    if (!kCand) {
      jj += G;
      if (jj >= units_per_row) {
        rr += (int)(jj / units_per_row);
        jj %= units_per_row;
      }
    } else {
      jj += j_step;
      if (jj >= units_per_row) {
        rr += row_step;
        jj = j0;
      }
    }
    if (rr > R) rr = R;
  };
  auto tile_of = [&](int64_t jj) -> int64_t { return jj * kUnitTiles + 4 * wave; };

  struct Unit {
    i32x8 b[kUnroll];
    bool ok[kUnroll][2];
  };
  auto fetch = [&](int rr, int64_t jj, Unit& x) {
    const int64_t t0 = tile_of(jj);
    const int seq = row_seq ? row_seq[rr] : rr;
    const int64_t limit = row_limit ? row_limit[rr] : T - 1;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      // a tile never straddles a page: one translation per tile
      const int64_t p0 = (t0 + i) * kTile;
      const int64_t row0 = p0 >= T ? -1 : (kPaged ? phys_row(pm, seq, T, p0) : (int64_t)seq * T + p0);
      const uint8_t* kp = k_idx + (row0 + kn) * kIndexDim + part;
      uint4 v[2];
      if (row0 >= 0 && p0 + kTile <= T && p0 + kTile - 1 <= limit) {
        // the whole tile is visible (the wave-uniform common case)
        x.ok[i][0] = x.ok[i][1] = true;
        v[0] = load_key_part<kCand>(kp);
        v[1] = load_key_part<kCand>(kp + 16 * kIndexDim);
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t p = p0 + 16 * hh + kn;
          x.ok[i][hh] = row0 >= 0 && p < T && p <= limit;
          v[hh] = x.ok[i][hh] ? load_key_part<kCand>(kp + 16 * hh * kIndexDim) : make_uint4(0, 0, 0, 0);
        }
      }
      x.b[i] = tile_pair(v[0], v[1]);
    }
  };
  // the same loads with no branch: a masked half reads key row 0 of the array and is left as loaded (its
  // score only lands in its own output column, which the ok flag discards; zeroing the loaded registers would
  // wait for the load).  The prologue's sample keys, issued first, can then be waited for alone while the
  // unit's keys are in flight.
  auto fetch_flat = [&](int rr, int64_t jj, Unit& x) {
    const int64_t t0 = tile_of(jj);
    const int seq = row_seq ? row_seq[rr] : rr;
    const int64_t limit = row_limit ? row_limit[rr] : T - 1;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const int64_t p0 = (t0 + i) * kTile;
      const int64_t row0 = p0 >= T ? -1 : (kPaged ? phys_row(pm, seq, T, p0) : (int64_t)seq * T + p0);
      uint4 v[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int64_t p = p0 + 16 * hh + kn;
        x.ok[i][hh] = row0 >= 0 && p < T && p <= limit;
        v[hh] = load_key_part<kCand>(k_idx + (x.ok[i][hh] ? row0 + 16 * hh + kn : 0) * kIndexDim + part);
      }
      x.b[i] = tile_pair(v[0], v[1]);
    }
  };
  uint32_t tau = 0, sh = 0;
  float tf = 0.f;
  auto query = [&](int rr, f16x8* a) {
    query_operands(q_idx + (int64_t)rr * kIndexDim, lane, a);
    if (kCand) {
      tau = uniform_u32(cand.row[rr].tau_s);
      sh = uniform_u32(cand.row[rr].sh);
      // the candidate test on the float score: key(s) >= tau_s exactly when s >= key_score(tau_s) (NaN and -inf
      // fail both; with tau_s = 0 every finite score passes); the key itself is formed only for candidates
      tf = tau ? key_score(tau) : -3.402823466e38f;
    }
  };
  auto wave_flush = [&](int rr) {
    uint2* base = cand.kp + (int64_t)rr * T;
    for (uint32_t e = lane; e < n_st; e += 64) base[s_dst[wave][e]] = s_ent[wave][e];
    n_st = 0;
  };
  auto flush = [&](int rr) {
    wave_flush(rr);
    __syncthreads();
    uint32_t* g = cand.hist + (int64_t)rr * kStreamHistWords;
    for (int i = threadIdx.x; i < kStreamBins; i += 256) {
      const uint32_t v = h[i];
      if (v) {
        atomicAdd(&g[i], v);
        h[i] = 0u;
      }
    }
    __syncthreads();
  };

  if (kCand) {
    for (int i = threadIdx.x; i < kStreamBins; i += 256) h[i] = 0u;
    __syncthreads();
  }
  Unit cur, nxt;
  f16x8 a[2];
  if (kCand && cand.samp) {
    // every workgroup serves one row (R <= G): the row's threshold from its sample, derived alike by each of
    // the row's workgroups; the one holding the row's first unit records it for the selection passes
    uint32_t skey[kSamplePer];
    sample_load_256(cand.samp + (int64_t)r * kSampleN, skey);
    fetch_flat(r, j, cur);
    query_operands(q_idx + (int64_t)r * kIndexDim, lane, a);
    const int64_t limit = row_limit ? row_limit[r] : T - 1;
    const int64_t V = limit < 0 ? 0 : (limit + 1 < T ? limit + 1 : T);
    uint32_t t_s, s_h;
    sample_threshold_256(skey, V, cand.k, h, s_wt, s_res, t_s, s_h);
    tau = uniform_u32(t_s);
    sh = uniform_u32(s_h);
    tf = tau ? key_score(tau) : -3.402823466e38f;
    if (j == 0 && threadIdx.x == 0) {
      cand.row[r].tau_s = tau;
      cand.row[r].sh = sh;
    }
  } else {
    fetch(r, j, cur);
    query(r, a);
  }
  while (r < R) {
    int rn = r;
    int64_t jn = j;
    advance(rn, jn);
    if (rn < R) fetch(rn, jn, nxt);
    const int64_t t0 = tile_of(j);
    float* out = scores ? scores + (int64_t)r * T : nullptr;
    float key[kUnroll][2];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const float2 sc = mfma_score(a, cur.b[i]);
      const float sv[2] = {sc.x, sc.y};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int64_t p = (t0 + i) * kTile + 16 * hh + kn;
        key[i][hh] = (kCand && lane < 16 && cur.ok[i][hh]) ? sv[hh] : -__builtin_inff();
        if (kOut && lane < 16 && p < T) out[p] = cur.ok[i][hh] ? sv[hh] : neg_inf;
      }
    }
    if (kCand) {
      // this wave's block: 4 j + wave, positions [128 (4 j + wave), + 128)
      const int64_t blk = 4 * j + wave;
      if (n_st + kBlockPositions > (uint32_t)kStage) wave_flush(r);
      uint32_t at = 0;
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bool c = key[i][hh] >= tf;
          const uint64_t m = __ballot(c);
          if (c) {
            const uint32_t kk = score_key(key[i][hh]);
            const uint32_t o = at + lanes_below(m);
            s_ent[wave][n_st + o] = make_uint2(kk, (uint32_t)((t0 + i) * kTile + 16 * hh + kn));
            s_dst[wave][n_st + o] = (uint32_t)(blk * kBlockPositions) + o;
            atomicAdd(&h[min((kk - tau) >> sh, (uint32_t)(kStreamBins - 1))], 1u);
          }
          at += (uint32_t)__popcll(m);
        }
      }
      n_st += at;
      if (lane == 0) cand.cnt[(int64_t)r * cand.n_blocks + blk] = at;
    }
    if (rn != r) {
      if (kCand) flush(r);
      if (rn < R) query(rn, a);
    }
    r = rn;
    j = jn;
    cur = nxt;
  }
}

// Candidate threshold of the streaming pool selection, in two kernels.
//
// Sample: S = 4096 keys per row in 512 runs of 8 adjacent positions; run u
// starts at ((2u + 1) V) / 1024 - 4 (clamped to the visible range [0, V),
// V = min(T, row_limit + 1)), so the runs cover the row evenly and each costs
// one 512-byte read.  Each wave scores kSampleTiles 32-sample tiles with the
// scan's tile arithmetic (two for a few rows, four for many: fewer, longer
// workgroups, -15 us at 4,096 rows); the keys go to samp [R][S].  Grid
// (S / (128 kSampleTiles), R).  Given hist (when no threshold kernel runs),
// the row's workgroups also clear its histogram and selection state for the
// scan.

template <int kSampleTiles, bool kPaged>
__global__ void __launch_bounds__(256)
index_sample_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                    uint32_t* __restrict__ samp, StreamRow* __restrict__ rows, uint32_t* __restrict__ hist,
                    PageMap pm) {
  const int r = blockIdx.y, tid = threadIdx.x;
  if (hist) {
    uint4* hr = reinterpret_cast<uint4*>(hist + (int64_t)r * kStreamHistWords);
    for (int i = blockIdx.x * 256 + tid; i < kStreamHistWords / 4; i += gridDim.x * 256) hr[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && tid == 0) rows[r] = StreamRow{};
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int kn = lane & 15, part = 16 * (lane >> 4);
  const int64_t limit = row_limit ? row_limit[r] : T - 1;
  const int64_t V = limit < 0 ? 0 : (limit + 1 < T ? limit + 1 : T);
  const int seq = row_seq ? row_seq[r] : r;
  constexpr int kRuns = kSampleN / kSampleRun;
  i32x8 kb[kSampleTiles];
  bool ok[kSampleTiles][2];
  // rows first, then every load unconditional (key row 0 where masked): a load under a branch, or after a
  // page-table branch, made the compiler wait for each before issuing the next
  int64_t rw[kSampleTiles][2];
#pragma unroll
  for (int u = 0; u < kSampleTiles; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int64_t i = ((int64_t)(blockIdx.x * 4 + wave) * kSampleTiles + u) * kTile + 16 * hh + kn;
      const int64_t run = i / kSampleRun;
      int64_t p0 = ((2 * run + 1) * V) / (2 * kRuns) - kSampleRun / 2;
      p0 = p0 < 0 ? 0 : (p0 > V - kSampleRun ? V - kSampleRun : p0);
      int64_t p = p0 + i % kSampleRun;
      p = p < 0 ? 0 : (p >= V ? V - 1 : p);
      rw[u][hh] = V <= 0 ? -1 : (kPaged ? phys_row(pm, seq, T, p) : (int64_t)seq * T + p);
      ok[u][hh] = rw[u][hh] >= 0;
    }
  // the query with the keys, in the same round trip
  f16x8 a[2];
  query_operands(q_idx + (int64_t)r * kIndexDim, lane, a);
  uint4 v[kSampleTiles][2];
#pragma unroll
  for (int u = 0; u < kSampleTiles; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) v[u][hh] = load_key_part(k_idx + (ok[u][hh] ? rw[u][hh] : 0) * kIndexDim + part);
#pragma unroll
  for (int u = 0; u < kSampleTiles; ++u) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      if (!ok[u][hh]) v[u][hh] = make_uint4(0, 0, 0, 0);
    kb[u] = tile_pair(v[u][0], v[u][1]);
  }
#pragma unroll
  for (int u = 0; u < kSampleTiles; ++u) {
    const float2 sc = mfma_score(a, kb[u]);
    const int64_t i = ((int64_t)(blockIdx.x * 4 + wave) * kSampleTiles + u) * kTile + kn;
    if (lane < 16) {
      samp[(int64_t)r * kSampleN + i] = ok[u][0] ? score_key(sc.x) : 0u;
      samp[(int64_t)r * kSampleN + i + 16] = ok[u][1] ? score_key(sc.y) : 0u;
    }
  }
}

// Threshold: one 1024-thread workgroup per row.  tau_s is the lower edge of
// the 22-bit key prefix holding the m-th largest sample key, m = ceil(mu +
// 4 sqrt(mu) + 8) with mu = k S / V: about m V / S positions score at or above
// it, at least k unless the sample misleads by four standard deviations (the
// selection checks the count and recovers).  tau_s = 0 (every visible
// position) when m > S.  The candidate histogram's digit shift sh puts the
// sample's largest key at digit < 2048.  Also clears the row's histogram and
// selection state before the scan.

__global__ void __launch_bounds__(1024)
index_tau_kernel(const uint32_t* __restrict__ samp, int64_t T, const int64_t* __restrict__ row_limit, int32_t k,
                 StreamRow* __restrict__ rows, uint32_t* __restrict__ hist) {
  constexpr int kBins = 4096;
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t wt[16];
  __shared__ uint32_t res[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t limit = row_limit ? row_limit[r] : T - 1;
  const int64_t V = limit < 0 ? 0 : (limit + 1 < T ? limit + 1 : T);
  for (int i = tid; i < kStreamHistWords; i += 1024) hist[(int64_t)r * kStreamHistWords + i] = 0u;
  const uint32_t m = sample_rank(k, V);
  if (m == 0u) {
    if (tid == 0) {
      StreamRow st = {};
      st.tau_s = 0u;
      st.sh = 21u;           // (key >> 21) < 2048 for every key
      rows[r] = st;
    }
    return;
  }
  constexpr int kPer = kSampleN / 1024;
  const uint4 kv = *reinterpret_cast<const uint4*>(samp + (int64_t)r * kSampleN + 4 * tid);
  const uint32_t key[kPer] = {kv.x, kv.y, kv.z, kv.w};
  for (int i = tid; i < kBins; i += 1024) h[i] = 0u;
  __syncthreads();
  uint32_t kmax = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    kmax = max(kmax, key[j]);
    atomicAdd(&h[key[j] >> 20], 1u);
  }
  __syncthreads();
  uint32_t need = m;
  find_bin_1024<kBins>(h, need, wt, res);
  __syncthreads();
  uint32_t prefix = res[0] << 20;
  need -= res[1];
  __syncthreads();
  h[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if ((key[j] >> 20) == (prefix >> 20)) atomicAdd(&h[(key[j] >> 10) & 1023u], 1u);
  __syncthreads();
  find_bin_1024<1024>(h, need, wt, res);
  __syncthreads();
  prefix |= res[0] << 10;
  // the sample's largest key
  kmax = wave_max_u32(kmax);
  if (lane == 0) wt[wave] = kmax;
  __syncthreads();
  if (tid == 0) {
    uint32_t mx = 0u;
    for (int w = 0; w < 16; ++w) mx = max(mx, wt[w]);
    const uint32_t span = mx - prefix;      // mx >= prefix: prefix is at most a sample key
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    StreamRow st = {};
    st.tau_s = prefix;
    st.sh = (uint32_t)(bits > 11 ? bits - 11 : 0);
    rows[r] = st;
  }
}

// Up to 32 query rows per workgroup (grid.y = ceil(R/32)): chunked prefill.
// Rows of one workgroup that share a sequence are scored together; a
// workgroup whose rows span several sequences handles one sequence at a time.
__global__ void __launch_bounds__(256)
index_block_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int R, int64_t T,
                   const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                   float* __restrict__ scores, int tiles_per_block) {
  __shared__ int s_seq[32];
  __shared__ int64_t s_lim[32];
  const int r0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kn = lane & 15, g = lane >> 4;
  if (threadIdx.x < 32) {
    int r = r0 + threadIdx.x;
    s_seq[threadIdx.x] = r < R ? (row_seq ? row_seq[r] : r) : -1;
    s_lim[threadIdx.x] = r < R ? (row_limit ? row_limit[r] : T - 1) : -1;
  }
  __syncthreads();

  const int64_t n_tiles = (T + kTile - 1) / kTile;
  const int64_t t_begin = (int64_t)blockIdx.x * tiles_per_block;
  const int64_t t_end = min(n_tiles, t_begin + tiles_per_block);
  const float neg_inf = -__builtin_inff();

  uint32_t done = 0;
  for (int m = 0; m < 32; ++m)
    if (s_seq[m] < 0) done |= 1u << m;

  while (done != 0xFFFFFFFFu) {
    int first = __builtin_ctz(~done);
    const int seq = s_seq[first];
    uint32_t active = 0;
    for (int m = 0; m < 32; ++m)
      if (!(done >> m & 1u) && s_seq[m] == seq) active |= 1u << m;
    done |= active;
    // the largest visible position among the active rows bounds the useful tiles
    int64_t max_lim = -1;
    for (int m = 0; m < 32; ++m)
      if (active >> m & 1u) max_lim = max(max_lim, s_lim[m]);

    // A operands of the two 16-row halves: lane 16 g + m holds bytes 16 g ..
    // 16 g + 15 of query row 16 mt + m (the decode layout with every row filled)
    f16x8 a[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (active >> (16 * mt + kn) & 1u)
        x = *reinterpret_cast<const uint4*>(q_idx + (int64_t)(r0 + 16 * mt + kn) * kIndexDim + 16 * g);
      fp8x16_to_f16(x.x, x.y, x.z, x.w, a[mt]);
    }
    const uint8_t* kseq = k_idx + (int64_t)seq * T * kIndexDim;

    for (int64_t t0 = t_begin + wave; t0 < t_end; t0 += 4 * kUnroll) {
      i32x8 b[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t t = t0 + 4 * u;
        uint4 v[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t c = t * kTile + 16 * hh + kn;
          v[hh] = (t < t_end && c < T && t * kTile <= max_lim) ? load_key_part(kseq + c * kIndexDim + 16 * g)
                                                                 : make_uint4(0, 0, 0, 0);
        }
        b[u] = tile_pair(v[0], v[1]);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t t = t0 + 4 * u;
        if (t >= t_end) break;
        f16x8 kb[2][2];
        fp8x16_to_f16((uint32_t)b[u][0], (uint32_t)b[u][1], (uint32_t)b[u][2], (uint32_t)b[u][3], kb[0]);
        fp8x16_to_f16((uint32_t)b[u][4], (uint32_t)b[u][5], (uint32_t)b[u][6], (uint32_t)b[u][7], kb[1]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (t * kTile <= max_lim) {
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][0], kb[hh][0], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][1], kb[hh][1], acc, 0, 0, 0);
            }
            const int64_t c = t * kTile + 16 * hh + kn;
            if (c < T) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int m = 16 * mt + 4 * g + i;
                if ((active >> m & 1u) && r0 + m < R)
                  scores[(int64_t)(r0 + m) * T + c] = c <= s_lim[m] ? acc[i] : neg_inf;
              }
            }
          }
        }
      }
    }
  }
}

// Query-block candidate scan: the rows of index_block_kernel (up to 32 per
// workgroup, rows of one sequence scored together) with the candidate output
// of index_stream_kernel in place of the scores.  Workgroup x covers the
// candidate blocks [x bpc, (x + 1) bpc) (bsz positions each), wave w the
// blocks x bpc + w, + 4, ..., each block's tiles in order.  The products take
// the keys as the A operand and the queries as B; the two 16-key halves of a
// 32-key tile interleave by fours (half hh holds positions 8 i + 4 hh + 0..3,
// i = 0..3), so lane 16 g + n ends up with the eight consecutive positions
// 8 g .. 8 g + 7 of the tile for query row n: a lane tests eight scores of one
// row, the row's four lanes (n, n + 16, n + 32, n + 48) order their candidates
// with two lane-pair exchanges per tile, and the row's running count for the
// block stays in a register.  The dot products are the same as with the
// operands the other way round.
constexpr int kCandUnroll = 2;     // tiles in flight per wave

// v of lane l ^ 16 and of lane l ^ 32 (the swaps leave the lane's own value
// and its partner's, in some order)
__device__ __forceinline__ uint32_t lane_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return r[0] + r[1] - v;
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] + r[1] - v;
}

template <bool kPaged, bool kOut>
__global__ void __launch_bounds__(256, 4)
index_block_cand_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int R, int64_t T,
                        const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                        float* __restrict__ scores, CandOut cand, int bsz, int bpc, PageMap pm) {
  __shared__ int s_seq[32];
  __shared__ int s_lim[32];
  __shared__ float s_tf[32];
  const int r0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kn = lane & 15, g = lane >> 4;
  if (threadIdx.x < 32) {
    const int r = r0 + threadIdx.x;
    int64_t lim = r < R ? (row_limit ? row_limit[r] : T - 1) : -1;
    lim = lim < -1 ? -1 : (lim > T - 1 ? T - 1 : lim);
    s_seq[threadIdx.x] = r < R ? (row_seq ? row_seq[r] : r) : -1;
    s_lim[threadIdx.x] = (int)lim;
    float tf = 0.f;
    if (r < R) {
      // as in the streaming scan: score >= key_score(tau_s) exactly when its key >= tau_s
      const uint32_t tau = cand.row[r].tau_s;
      tf = tau ? key_score(tau) : -3.402823466e38f;
    }
    s_tf[threadIdx.x] = tf;
  }
  __syncthreads();

  const int64_t blk_begin = (int64_t)blockIdx.x * bpc;
  const int64_t blk_end = min(cand.n_blocks, blk_begin + bpc);
  const int tiles_per_blk = bsz / kTile;
  const int Ti = (int)T;
  const float neg_inf = -__builtin_inff();

  uint32_t done = 0;
  for (int m = 0; m < 32; ++m)
    if (s_seq[m] < 0) done |= 1u << m;

  while (done != 0xFFFFFFFFu) {
    const int first = __builtin_ctz(~done);
    const int seq = s_seq[first];
    uint32_t active = 0;
    for (int m = 0; m < 32; ++m)
      if (!(done >> m & 1u) && s_seq[m] == seq) active |= 1u << m;
    done |= active;
    int max_lim = -1, min_lim = Ti;
    for (int m = 0; m < 32; ++m)
      if (active >> m & 1u) {
        max_lim = max(max_lim, s_lim[m]);
        min_lim = min(min_lim, s_lim[m]);
      }

    // B operands: lane 16 g + n holds bytes 16 g .. 16 g + 15 of query row 16 mt + n
    f16x8 a[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (active >> (16 * mt + kn) & 1u)
        x = *reinterpret_cast<const uint4*>(q_idx + (int64_t)(r0 + 16 * mt + kn) * kIndexDim + 16 * g);
      fp8x16_to_f16(x.x, x.y, x.z, x.w, a[mt]);
    }
    // the lane's rows 16 mt + n: liveness, limit (-1: none visible), threshold, candidate row
    bool live[2];
    int lim[2];
    float tf[2];
    uint2* kp_row[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int m = 16 * mt + kn;
      live[mt] = active >> m & 1u;
      lim[mt] = live[mt] ? s_lim[m] : -1;
      tf[mt] = s_tf[m];
      kp_row[mt] = cand.kp + (int64_t)(r0 + m) * T;
    }

    for (int64_t blk = blk_begin + wave; blk < blk_end; blk += 4) {
      uint32_t at[2] = {0u, 0u};
      const int pb = (int)(blk * bsz);
      if (kOut || pb <= max_lim) {
        for (int t = 0; t < tiles_per_blk; t += kCandUnroll) {
          i32x8 b[kCandUnroll];
          bool mapped[kCandUnroll];
#pragma unroll
          for (int u = 0; u < kCandUnroll; ++u) {
            const int p0 = pb + (t + u) * kTile;
            int64_t row0 = -1;
            if (p0 <= max_lim) row0 = kPaged ? phys_row(pm, seq, T, p0) : (int64_t)seq * T + p0;
            mapped[u] = row0 >= 0;
            uint4 v[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int off = 8 * (kn >> 2) + 4 * hh + (kn & 3);
              v[hh] = (row0 >= 0 && p0 + off < Ti)
                          ? load_key_part<false>(k_idx + (row0 + off) * kIndexDim + 16 * g)
                          : make_uint4(0, 0, 0, 0);
            }
            b[u] = tile_pair(v[0], v[1]);
          }
#pragma unroll
          for (int u = 0; u < kCandUnroll; ++u) {
            const int p0 = pb + (t + u) * kTile;
            if (!kOut && p0 > max_lim) break;
            f16x8 kb[2][2];
            fp8x16_to_f16((uint32_t)b[u][0], (uint32_t)b[u][1], (uint32_t)b[u][2], (uint32_t)b[u][3], kb[0]);
            fp8x16_to_f16((uint32_t)b[u][4], (uint32_t)b[u][5], (uint32_t)b[u][6], (uint32_t)b[u][7], kb[1]);
            f32x4 acc[2][2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int mt = 0; mt < 2; ++mt) {
                acc[hh][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[hh][0], a[mt][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                acc[hh][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[hh][1], a[mt][1], acc[hh][mt], 0, 0, 0);
              }
            // lane 16 g + n holds positions pl .. pl + 7 of query row n: slot 4 hh + j is
            // acc[hh][.][j]; a tile fully mapped, inside T and visible to every active row (all
            // but the tiles at the causal edge) needs only the threshold test per score
            const int pl = p0 + 8 * g;
            const bool full = mapped[u] && p0 + kTile <= Ti && p0 + kTile - 1 <= min_lim;
            const int n_t = min(8, max(0, Ti - pl));
            const int n_in = mapped[u] ? n_t : 0;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
              const int n_vis = full ? (live[mt] ? 8 : 0) : min(n_in, max(0, lim[mt] - pl + 1));
              uint32_t m8 = 0;
              if (full) {
                if (live[mt]) {
#pragma unroll
                  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int j = 0; j < 4; ++j) m8 |= (uint32_t)(acc[hh][mt][j] >= tf[mt]) << (4 * hh + j);
                }
              } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    m8 |= (uint32_t)((4 * hh + j < n_vis) & (acc[hh][mt][j] >= tf[mt])) << (4 * hh + j);
              }
              // the row's four lanes in position order: g = 0, 1, 2, 3
              const uint32_t cnt = (uint32_t)__popc(m8);
              const uint32_t x16 = lane_xor16(cnt);
              const uint32_t pair = cnt + x16;
              const uint32_t x32 = lane_xor32(pair);
              uint32_t o = at[mt] + ((g & 1) ? x16 : 0u) + ((g & 2) ? x32 : 0u);
              at[mt] += pair + x32;
              while (m8) {
                const int sl = __builtin_ctz(m8);
                m8 &= m8 - 1u;
                const f32x4 h = sl < 4 ? acc[0][mt] : acc[1][mt];
                const int j = sl & 3;
                const float sv = j == 0 ? h[0] : (j == 1 ? h[1] : (j == 2 ? h[2] : h[3]));
                kp_row[mt][pb + o] = make_uint2(score_key(sv), (uint32_t)(pl + sl));
                ++o;
              }
              if (kOut && live[mt]) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    if (4 * hh + j < n_t)
                      scores[(int64_t)(r0 + 16 * mt + kn) * T + pl + 4 * hh + j] = 4 * hh + j < n_vis ? acc[hh][mt][j] : neg_inf;
              }
            }
          }
        }
      }
      if (g == 0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          if (live[mt]) cand.cnt[(int64_t)(r0 + 16 * mt + kn) * cand.n_blocks + blk] = at[mt];
      }
    }
  }
}

// workgroups of index_stream_kernel to launch: the resident count, at most 3
// per CU (3 beat 4 and 2 in a same-box sweep of the 8 x 1M candidate scan:
// 95.6 vs 98.4 and 102 us; more concurrent key streams than that contend)
static int64_t resident_blocks() {
  static std::atomic<int> per_cu_cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int per_cu = per_cu_cache[dev].load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(index_stream_kernel<true, false, false>), 256,
                                                      0) != hipSuccess || per_cu < 1)
      per_cu = 3;
    per_cu_cache[dev].store(per_cu, std::memory_order_relaxed);
  }
  return (int64_t)device_cu_count() * std::min(per_cu, 3);
}

static int tiles_per_block_for(int64_t n_tiles, int64_t rows) {
  // aim for >= ~2048 workgroups in total, at least 4 tiles (one per wave) each
  // (4 rather than 16 took 3 us off the 8 x 16,384 Reindex scan of the decode step)
  int64_t want_blocks_per_row = (2048 + rows - 1) / rows;
  int64_t tpb = (n_tiles + want_blocks_per_row - 1) / want_blocks_per_row;
  if (tpb < 4) tpb = 4;
  tpb = (tpb + 3) / 4 * 4;
  return (int)tpb;
}

void launch_index_scan(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T, const int32_t* row_seq,
                       const int64_t* row_limit, float* scores, const CandOut* cand, hipStream_t s,
                       const PageMap& pm) {
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  const int64_t units_per_row = (n_tiles + kUnitTiles - 1) / kUnitTiles;
  int64_t grid = std::min<int64_t>(resident_blocks(), (int64_t)R * units_per_row);
  if (cand && R <= grid) grid = std::min<int64_t>(grid / R, units_per_row) * R;   // whole groups per row
  const dim3 g((unsigned)grid), blk(256);
  const bool paged = pm.table != nullptr;
  if (cand) {
    const CandOut& c = *cand;
    if (paged) {
      if (scores) index_stream_kernel<true, true, true><<<g, blk, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R, units_per_row, c, pm);
      else index_stream_kernel<true, true, false><<<g, blk, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R, units_per_row, c, pm);
    } else {
      if (scores) index_stream_kernel<true, false, true><<<g, blk, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R, units_per_row, c, pm);
      else index_stream_kernel<true, false, false><<<g, blk, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R, units_per_row, c, pm);
    }
  } else if (paged) {
    index_stream_kernel<false, true, true><<<g, blk, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R, units_per_row, CandOut{}, pm);
  } else {
    index_stream_kernel<false, false, true><<<g, blk, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R, units_per_row, CandOut{}, pm);
  }
}

void launch_index_block_cand(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T,
                             const int32_t* row_seq, const int64_t* row_limit, float* scores, const CandOut& cand,
                             int bsz, hipStream_t s, const PageMap& pm) {
  // about 8,192 workgroups, at least 4 blocks (one per wave) each (8,192 beat
  // 2,048 by 7% at 4,096 x 262,144: shorter workgroups balance better); when
  // grid.x is a multiple of 8, the workgroups of one key range (same x, every
  // row group) land on one XCD and share its L2
  const int64_t row_groups = ((int64_t)R + 31) / 32;
  int64_t bpc = (cand.n_blocks * row_groups + 8191) / 8192;
  bpc = (std::max<int64_t>(bpc, 4) + 3) / 4 * 4;
  const dim3 grid((unsigned)((cand.n_blocks + bpc - 1) / bpc), (unsigned)row_groups), blk(256);
  const bool paged = pm.table != nullptr;
  if (paged) {
    if (scores) index_block_cand_kernel<true, true><<<grid, blk, 0, s>>>(q_idx, k_idx, R, T, row_seq, row_limit, scores, cand, bsz, (int)bpc, pm);
    else index_block_cand_kernel<true, false><<<grid, blk, 0, s>>>(q_idx, k_idx, R, T, row_seq, row_limit, scores, cand, bsz, (int)bpc, pm);
  } else {
    if (scores) index_block_cand_kernel<false, true><<<grid, blk, 0, s>>>(q_idx, k_idx, R, T, row_seq, row_limit, scores, cand, bsz, (int)bpc, pm);
    else index_block_cand_kernel<false, false><<<grid, blk, 0, s>>>(q_idx, k_idx, R, T, row_seq, row_limit, scores, cand, bsz, (int)bpc, pm);
  }
}

void launch_index_sample_tau(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T,
                             const int32_t* row_seq, const int64_t* row_limit, int32_t k, StreamRow* rows,
                             uint32_t* hist, uint32_t* samp, bool tau, hipStream_t s, const PageMap& pm) {
  // the threshold kernel clears the rows' state when it runs, the sample kernel otherwise
  uint32_t* clear = tau ? nullptr : hist;
  const dim3 g4(kSampleN / (4 * 4 * kTile), R), g2(kSampleN / (4 * 2 * kTile), R);
  if (pm.table) {
    if (R >= 64) index_sample_kernel<4, true><<<g4, 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, samp, rows, clear, pm);
    else index_sample_kernel<2, true><<<g2, 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, samp, rows, clear, pm);
  } else {
    if (R >= 64) index_sample_kernel<4, false><<<g4, 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, samp, rows, clear, pm);
    else index_sample_kernel<2, false><<<g2, 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, samp, rows, clear, pm);
  }
  if (tau) index_tau_kernel<<<R, 1024, 0, s>>>(samp, T, row_limit, k, rows, hist);
}

int64_t index_sample_words() { return kSampleN; }

int64_t index_scan_blocks(int64_t T) {
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  return (n_tiles + kUnitTiles - 1) / kUnitTiles * 4;
}

bool index_scan_streams(int32_t R, const int32_t* row_seq) { return !(row_seq && R >= 32); }

bool index_scan_derives_tau(int32_t R) { return (int64_t)R <= resident_blocks(); }

}  // namespace csa2

using namespace csa2;

extern "C" csa2_status csa2_index_full(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B,
                                       int64_t T, const int32_t* row_seq, const int64_t* row_limit,
                                       float* scores, void* stream) {
  if (!q_idx || !k_idx || !scores) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (T % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(scores, 16)) return CSA2_EALIGN;
  {
    const csa2_status dc = debug_check(row_seq, R, B, nullptr, nullptr, 0, 0, nullptr, 0, T, (hipStream_t)stream);
    if (dc != CSA2_OK) return dc;
  }
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  hipStream_t s = (hipStream_t)stream;
  if (!index_scan_streams(R, row_seq)) {
    int tpb = tiles_per_block_for(n_tiles, (R + 31) / 32);
    dim3 grid(ceil_div(n_tiles, tpb), ceil_div(R, 32));
    index_block_kernel<<<grid, 256, 0, s>>>(q_idx, k_idx, R, T, row_seq, row_limit, scores, tpb);
  } else {
    launch_index_scan(q_idx, k_idx, R, T, row_seq, row_limit, scores, nullptr, s, PageMap{});
  }
  return launch_status();
}

extern "C" csa2_status csa2_index_full_fp8(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B,
                                           int64_t T, const int32_t* row_seq, const int64_t* row_limit,
                                           float* scores, void* stream) {
  if (!q_idx || !k_idx || !scores) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (T % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(scores, 16)) return CSA2_EALIGN;
  {
    const csa2_status dc = debug_check(row_seq, R, B, nullptr, nullptr, 0, 0, nullptr, 0, T, (hipStream_t)stream);
    if (dc != CSA2_OK) return dc;
  }
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  const int tpb = tiles_per_block_for(n_tiles, R);
  const dim3 grid(ceil_div(n_tiles, tpb), R);
  index_rows_kernel<false, true><<<grid, 256, 0, (hipStream_t)stream>>>(q_idx, k_idx, T, row_seq, row_limit, nullptr,
                                                                        T, scores, tpb, PageMap{});
  return launch_status();
}

extern "C" csa2_status csa2_index_reindex(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B,
                                          int64_t T, const int32_t* row_seq, const int32_t* pool, int32_t P,
                                          float* scores, void* stream) {
  if (!q_idx || !k_idx || !scores || !pool) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0 || P <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (P % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(scores, 16) || !aligned(pool, 16)) return CSA2_EALIGN;
  {
    const csa2_status dc = debug_check(row_seq, R, B, nullptr, nullptr, 0, 0, nullptr, 0, T, (hipStream_t)stream);
    if (dc != CSA2_OK) return dc;
  }
  const int64_t n_tiles = (P + kTile - 1) / kTile;
  int tpb = tiles_per_block_for(n_tiles, R);
  dim3 grid(ceil_div(n_tiles, tpb), R);
  index_rows_kernel<true><<<grid, 256, 0, (hipStream_t)stream>>>(q_idx, k_idx, T, row_seq, nullptr, pool, P,
                                                                 scores, tpb, PageMap{});
  return launch_status();
}

csa2_status csa2::check_pages(const int32_t* block_table, int64_t max_blocks, int32_t page, int64_t T) {
  if (!block_table || max_blocks <= 0 || page <= 0) return CSA2_EINVAL;
  if (page % kPageQuantum != 0 || T > max_blocks * (int64_t)page) return CSA2_ESHAPE;
  return CSA2_OK;
}

extern "C" csa2_status csa2_index_full_paged(const uint8_t* q_idx, const uint8_t* k_pages, int32_t R, int32_t B,
                                             int64_t T, const int32_t* row_seq, const int64_t* row_limit,
                                             const int32_t* block_table, int64_t max_blocks, int32_t page,
                                             float* scores, void* stream) {
  if (!q_idx || !k_pages || !scores) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (T % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  csa2_status st = check_pages(block_table, max_blocks, page, T);
  if (st != CSA2_OK) return st;
  if (!aligned(q_idx, 16) || !aligned(k_pages, 16) || !aligned(scores, 16)) return CSA2_EALIGN;
  {
    const csa2_status dc = debug_check(row_seq, R, B, nullptr, nullptr, 0, 0, nullptr, 0, T, (hipStream_t)stream);
    if (dc != CSA2_OK) return dc;
  }
  launch_index_scan(q_idx, k_pages, R, T, row_seq, row_limit, scores, nullptr, (hipStream_t)stream,
                    PageMap{block_table, max_blocks, page});
  return launch_status();
}

extern "C" csa2_status csa2_index_reindex_paged(const uint8_t* q_idx, const uint8_t* k_pages, int32_t R, int32_t B,
                                                int64_t T, const int32_t* row_seq, const int32_t* block_table,
                                                int64_t max_blocks, int32_t page, const int32_t* pool, int32_t P,
                                                float* scores, void* stream) {
  if (!q_idx || !k_pages || !scores || !pool) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0 || P <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (P % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  csa2_status st = check_pages(block_table, max_blocks, page, T);
  if (st != CSA2_OK) return st;
  if (!aligned(q_idx, 16) || !aligned(k_pages, 16) || !aligned(scores, 16) || !aligned(pool, 16)) return CSA2_EALIGN;
  {
    const csa2_status dc = debug_check(row_seq, R, B, nullptr, nullptr, 0, 0, nullptr, 0, T, (hipStream_t)stream);
    if (dc != CSA2_OK) return dc;
  }
  const int64_t n_tiles = (P + kTile - 1) / kTile;
  int tpb = tiles_per_block_for(n_tiles, R);
  dim3 grid(ceil_div(n_tiles, tpb), R);
  index_rows_kernel<true, false, true><<<grid, 256, 0, (hipStream_t)stream>>>(q_idx, k_pages, T, row_seq, nullptr,
                                                                               pool, P, scores, tpb,
                                                                               PageMap{block_table, max_blocks, page});
  return launch_status();
}
