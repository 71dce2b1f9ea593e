// Indexer scoring kernels: Full mode (every visible position) and Reindex mode
// (only the candidate-pool positions), per the CSA2 roles paragraph of the
// MarkTechPost retelling of DeepSeek-V4.1-Flash.
//
// score(r, j) = sum_{d<64} q_idx[r][d] * k_idx[seq(r)][j][d] with E4M3 inputs.
// The E4M3 bytes are widened to f16 (exact, v_cvt_scalef32_pk_f16_fp8 with unit
// scale) and multiplied on the f16 matrix cores:
//   v_mfma_f32_32x32x16_f16:  C[32 x 32] += A[32 x 16] * B[16 x 32], four k-steps
// with A = up to 32 query rows of one sequence and B = 32 keys.  On gfx950 this
// instruction forms each 16-term dot product exactly and rounds it once into
// the fp32 accumulator, so a score carries at most four roundings (one per
// k-step, error <= 2^-22 * sum |q_d k_d|); whenever the running sums fit in 24
// bits -- as for unit-normal E4M3 inputs -- the score is the exact value
// rounded once.  (The fp8 matrix path is not used: its internal accumulation
// keeps only ~20 bits below the largest product.)  Lane l owns row/column
// (l % 32) and one 32-byte half of the 64-d
// key, so a wave loads a 2 KB tile of 32 consecutive keys with two 16-byte
// loads per lane (fully coalesced); A and B use the same lane->k map.
// Output C: lane l, register v holds column l % 32 and row
// 8*(v/4) + 4*(l/32) + (v%4); row 0 sits in register 0 of lanes 0-31, which
// store 32 consecutive scores as one 128-byte line.
//
// Decode (one query per sequence) is HBM-bound: 64 bytes of key per score; the
// matrix cores and the conversions use a small share of their peak.  Chunked
// prefill fills all 32 rows of A and is bound by the fp32 score writes.
#include <algorithm>

#include "internal.hpp"
#include "tile.hpp"

namespace csa2 {

// One query row per workgroup row (grid.y = R).  Used for decode (Full and
// Reindex).  kGather: column c of row r scores position pool[r][c].
template <bool kGather>
__global__ void __launch_bounds__(256)
index_rows_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                  const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                  const int32_t* __restrict__ pool, int64_t n_cols, float* __restrict__ scores,
                  int tiles_per_block, PageMap pm) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col_in_tile = lane & 31;
  const int seq = row_seq ? row_seq[r] : r;
  const int64_t limit = row_limit ? row_limit[r] : T - 1;
  float* out = scores + (int64_t)r * n_cols;
  const int32_t* prow = kGather ? pool + (int64_t)r * n_cols : nullptr;

  i32x8 araw = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col_in_tile == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(q_idx + (int64_t)r * kIndexDim + 32 * half);
    uint4 x = q[0], y = q[1];
    araw[0] = x.x; araw[1] = x.y; araw[2] = x.z; araw[3] = x.w;
    araw[4] = y.x; araw[5] = y.y; araw[6] = y.z; araw[7] = y.w;
  }
  f16x8 a[4];
  fp8x32_to_f16(araw, a);

  const int64_t n_tiles = (n_cols + kTile - 1) / kTile;
  const int64_t t_begin = (int64_t)blockIdx.x * tiles_per_block;
  const int64_t t_end = min(n_tiles, t_begin + tiles_per_block);
  const float neg_inf = -__builtin_inff();

  for (int64_t t0 = t_begin + wave; t0 < t_end; t0 += 4 * kUnroll) {
    i32x8 b[kUnroll];
    int64_t pos[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t t = t0 + 4 * u;
      int64_t c = t * kTile + col_in_tile;
      int64_t p = -1;
      if (t < t_end && c < n_cols) p = kGather ? (int64_t)prow[c] : c;
      ok[u] = p >= 0 && p < T && p <= limit;
      const int64_t row = ok[u] ? phys_row(pm, seq, T, p) : -1;
      ok[u] = row >= 0;
      pos[u] = c;
      b[u] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (ok[u]) b[u] = load_half_key(k_idx + row * kIndexDim + 32 * half);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t t = t0 + 4 * u;
      f32x16 acc = mfma_score(a, b[u]);
      if (t < t_end && half == 0 && pos[u] < n_cols) out[pos[u]] = ok[u] ? acc[0] : neg_inf;
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
//    LDS, keeps the list of bins it touched and adds those counts to the row's
//    histogram when it leaves the row (once per workgroup; with row-major
//    order every workgroup would flush at each row boundary, measured slower).
constexpr int kUnitTiles = 16;

template <bool kCand>
__global__ void __launch_bounds__(256)
index_stream_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                    float* __restrict__ scores, int R, int64_t units_per_row, CandOut cand, PageMap pm) {
  __shared__ uint32_t h[kCand ? kStreamBins : 1];
  __shared__ uint32_t used[kCand ? kStreamBins : 1];   // bins of h that are nonzero, in the order first hit
  __shared__ uint32_t n_used;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col_in_tile = lane & 31;
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
    bool ok[kUnroll];
  };
  auto fetch = [&](int rr, int64_t jj, Unit& x) {
    const int64_t t0 = tile_of(jj);
    const int seq = row_seq ? row_seq[rr] : rr;
    const int64_t limit = row_limit ? row_limit[rr] : T - 1;
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      // a tile never straddles a page: one translation per tile
      const int64_t p0 = (t0 + i) * kTile;
      const int64_t row0 = p0 < T ? phys_row(pm, seq, T, p0) : -1;
      const int64_t p = p0 + col_in_tile;
      x.ok[i] = row0 >= 0 && p < T && p <= limit;
      x.b[i] = x.ok[i] ? load_half_key<kCand>(k_idx + (row0 + col_in_tile) * kIndexDim + 32 * half)
                       : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };
  uint32_t tau = 0, sh = 0;
  auto query = [&](int rr, f16x8* a) {
    i32x8 araw = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col_in_tile == 0) {
      const uint4* q = reinterpret_cast<const uint4*>(q_idx + (int64_t)rr * kIndexDim + 32 * half);
      const uint4 x = q[0], y = q[1];
      araw[0] = x.x; araw[1] = x.y; araw[2] = x.z; araw[3] = x.w;
      araw[4] = y.x; araw[5] = y.y; araw[6] = y.z; araw[7] = y.w;
    }
    fp8x32_to_f16(araw, a);
    if (kCand) {
      tau = uniform_u32(cand.row[rr].tau_s);
      sh = uniform_u32(cand.row[rr].sh);
    }
  };
  auto flush = [&](int rr) {
    __syncthreads();
    uint32_t* g = cand.hist + (int64_t)rr * kStreamHistWords;
    const uint32_t n = n_used;
    for (uint32_t i = threadIdx.x; i < n; i += 256) {
      const uint32_t bin = used[i];
      atomicAdd(&g[bin], h[bin]);
      h[bin] = 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) n_used = 0u;   // every thread has read n_used before the barrier above
    __syncthreads();
  };

  if (kCand) {
    for (int i = threadIdx.x; i < kStreamBins; i += 256) h[i] = 0u;
    if (threadIdx.x == 0) n_used = 0u;
    __syncthreads();
  }
  Unit cur, nxt;
  fetch(r, j, cur);
  f16x8 a[4];
  query(r, a);
  while (r < R) {
    int rn = r;
    int64_t jn = j;
    advance(rn, jn);
    if (rn < R) fetch(rn, jn, nxt);
    const int64_t t0 = tile_of(j);
    float* out = scores ? scores + (int64_t)r * T : nullptr;
    uint32_t key[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const f32x16 acc = mfma_score(a, cur.b[i]);
      const int64_t p = (t0 + i) * kTile + col_in_tile;
      key[i] = 0u;
      if (half == 0 && p < T) {
        if (!kCand || scores) out[p] = cur.ok[i] ? acc[0] : neg_inf;
        if (kCand && cur.ok[i]) key[i] = score_key(acc[0]);
      }
    }
    if (kCand) {
      // this wave's block: 4 j + wave, positions [128 (4 j + wave), + 128)
      const int64_t blk = 4 * j + wave;
      uint2* oc = cand.kp + (int64_t)r * T + blk * kBlockPositions;
      uint32_t at = 0;
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
        const bool c = key[i] != 0u && key[i] >= tau;
        const uint64_t m = __ballot(c);
        if (c) {
          const uint32_t o = at + lanes_below(m);
          oc[o] = make_uint2(key[i], (uint32_t)((t0 + i) * kTile + col_in_tile));
          const uint32_t bin = min((key[i] - tau) >> sh, (uint32_t)(kStreamBins - 1));
          if (atomicAdd(&h[bin], 1u) == 0u) used[atomicAdd(&n_used, 1u)] = bin;
        }
        at += (uint32_t)__popcll(m);
      }
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
// one 512-byte read.  Each wave scores two 32-sample tiles with the scan's
// tile arithmetic; the keys go to samp [R][S].  Grid (S / 256, R).
constexpr int kSampleN = 4096;
constexpr int kSampleRun = 8;

__global__ void __launch_bounds__(256)
index_sample_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                    const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit,
                    uint32_t* __restrict__ samp, PageMap pm) {
  const int r = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col_in_tile = lane & 31;
  const int64_t limit = row_limit ? row_limit[r] : T - 1;
  const int64_t V = limit < 0 ? 0 : (limit + 1 < T ? limit + 1 : T);
  const int seq = row_seq ? row_seq[r] : r;
  constexpr int kRuns = kSampleN / kSampleRun;
  i32x8 kb[2];
  bool ok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t i = ((int64_t)(blockIdx.x * 4 + wave) * 2 + u) * kTile + col_in_tile;
    const int64_t run = i / kSampleRun;
    int64_t p0 = ((2 * run + 1) * V) / (2 * kRuns) - kSampleRun / 2;
    p0 = p0 < 0 ? 0 : (p0 > V - kSampleRun ? V - kSampleRun : p0);
    int64_t p = p0 + i % kSampleRun;
    p = p < 0 ? 0 : (p >= V ? V - 1 : p);
    const int64_t row = V > 0 ? phys_row(pm, seq, T, p) : -1;
    ok[u] = row >= 0;
    kb[u] = ok[u] ? load_half_key(k_idx + row * kIndexDim + 32 * half) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  i32x8 araw = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col_in_tile == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(q_idx + (int64_t)r * kIndexDim + 32 * half);
    const uint4 x = q[0], y = q[1];
    araw[0] = x.x; araw[1] = x.y; araw[2] = x.z; araw[3] = x.w;
    araw[4] = y.x; araw[5] = y.y; araw[6] = y.z; araw[7] = y.w;
  }
  f16x8 a[4];
  fp8x32_to_f16(araw, a);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const f32x16 acc = mfma_score(a, kb[u]);
    const int64_t i = ((int64_t)(blockIdx.x * 4 + wave) * 2 + u) * kTile + col_in_tile;
    if (half == 0) samp[(int64_t)r * kSampleN + i] = ok[u] ? score_key(acc[0]) : 0u;
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
__device__ __forceinline__ uint32_t sample_rank(int32_t k, int64_t V) {
  if (V <= 0) return 0u;
  const double mu = (double)k * (double)kSampleN / (double)V;
  const double m = ceil(mu + 4.0 * sqrt(mu) + 8.0);
  return m > (double)kSampleN ? 0u : (uint32_t)m;
}

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
  const int half = lane >> 5;
  const int l32 = lane & 31;
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

  // rows m held by this lane's output registers
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

    i32x8 araw = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active >> l32 & 1u) {
      const uint4* q = reinterpret_cast<const uint4*>(q_idx + (int64_t)(r0 + l32) * kIndexDim + 32 * half);
      uint4 x = q[0], y = q[1];
      araw[0] = x.x; araw[1] = x.y; araw[2] = x.z; araw[3] = x.w;
      araw[4] = y.x; araw[5] = y.y; araw[6] = y.z; araw[7] = y.w;
    }
    f16x8 a[4];
    fp8x32_to_f16(araw, a);
    const uint8_t* kseq = k_idx + (int64_t)seq * T * kIndexDim;

    for (int64_t t0 = t_begin + wave; t0 < t_end; t0 += 4 * kUnroll) {
      i32x8 b[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int64_t t = t0 + 4 * u;
        int64_t c = t * kTile + l32;
        b[u] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (t < t_end && c < T && t * kTile <= max_lim) b[u] = load_half_key(kseq + c * kIndexDim + 32 * half);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int64_t t = t0 + 4 * u;
        if (t >= t_end) break;
        int64_t c = t * kTile + l32;
        f32x16 acc = {};
        if (t * kTile <= max_lim) acc = mfma_score(a, b[u]);
        if (c < T) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            int m = 8 * (v >> 2) + 4 * half + (v & 3);
            if ((active >> m & 1u) && r0 + m < R) {
              float s = c <= s_lim[m] ? acc[v] : neg_inf;
              scores[(int64_t)(r0 + m) * T + c] = s;
            }
          }
        }
      }
    }
  }
}

// workgroups of index_stream_kernel the device keeps resident at once
static int64_t resident_blocks() {
  static int64_t cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
        hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(index_stream_kernel<true>), 256,
                                                      0) != hipSuccess || per_cu < 1)
      per_cu = 4;
    cached = (int64_t)cus * per_cu;
  }
  return cached;
}

static int tiles_per_block_for(int64_t n_tiles, int64_t rows) {
  // aim for >= ~2048 workgroups in total, at least 16 tiles (2 KB/wave-tile) each
  int64_t want_blocks_per_row = (2048 + rows - 1) / rows;
  int64_t tpb = (n_tiles + want_blocks_per_row - 1) / want_blocks_per_row;
  if (tpb < 16) tpb = 16;
  tpb = (tpb + 15) / 16 * 16;
  return (int)tpb;
}

void launch_index_scan(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T, const int32_t* row_seq,
                       const int64_t* row_limit, float* scores, const CandOut* cand, hipStream_t s,
                       const PageMap& pm) {
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  const int64_t units_per_row = (n_tiles + kUnitTiles - 1) / kUnitTiles;
  int64_t grid = std::min<int64_t>(resident_blocks(), (int64_t)R * units_per_row);
  if (cand && R <= grid) grid = std::min<int64_t>(grid / R, units_per_row) * R;   // whole groups per row
  if (cand)
    index_stream_kernel<true><<<(int)grid, 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R,
                                                        units_per_row, *cand, pm);
  else
    index_stream_kernel<false><<<(int)grid, 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, scores, R,
                                                         units_per_row, CandOut{}, pm);
}

void launch_index_sample_tau(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T,
                             const int32_t* row_seq, const int64_t* row_limit, int32_t k, StreamRow* rows,
                             uint32_t* hist, uint32_t* samp, hipStream_t s, const PageMap& pm) {
  index_sample_kernel<<<dim3(kSampleN / 256, R), 256, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, samp, pm);
  index_tau_kernel<<<R, 1024, 0, s>>>(samp, T, row_limit, k, rows, hist);
}

int64_t index_sample_words() { return kSampleN; }

int64_t index_scan_blocks(int64_t T) {
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  return (n_tiles + kUnitTiles - 1) / kUnitTiles * 4;
}

bool index_scan_streams(int32_t R, const int32_t* row_seq) { return !(row_seq && R >= 32); }

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

extern "C" csa2_status csa2_index_reindex(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B,
                                          int64_t T, const int32_t* row_seq, const int32_t* pool, int32_t P,
                                          float* scores, void* stream) {
  if (!q_idx || !k_idx || !scores || !pool) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0 || P <= 0) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (P % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(scores, 16) || !aligned(pool, 16)) return CSA2_EALIGN;
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
  const int64_t n_tiles = (P + kTile - 1) / kTile;
  int tpb = tiles_per_block_for(n_tiles, R);
  dim3 grid(ceil_div(n_tiles, tpb), R);
  index_rows_kernel<true><<<grid, 256, 0, (hipStream_t)stream>>>(q_idx, k_pages, T, row_seq, nullptr, pool, P,
                                                                 scores, tpb, PageMap{block_table, max_blocks, page});
  return launch_status();
}
