// Top-K selection by radix select over order-preserving 32-bit keys.
//
// The HN summary's key points describe CSA2 layers sharing one set of Top-K
// indices and a shallow-layer candidate pool that bounds the deeper layers'
// search; the MarkTechPost retelling (CSA2 paragraph) bounds that pool at
// 16,384 positions.  Selection rule: the k largest visible scores, equal scores
// to the lower slot, output ascending, -1 padding.
//
// Each score maps to a key that orders like the float (sign flip for
// positives, bitwise not for negatives, -0 as +0); invisible slots (-inf, NaN,
// or a negative index_map entry) map to key 0, which no visible score reaches
// (the smallest, -FLT_MAX, maps to 0x00800000).  The k-th largest key tau is
// found digit by digit (11, 11 and 10 bits) with histograms; the output is
// then written in slot order (so it is sorted without a sort), taking every
// key > tau and the lowest-slot keys == tau.  All integer work: deterministic.
//
// Three paths, chosen on the host from the row length N:
//   small   (N <= 32768): one 1024-thread workgroup per row, keys in
//           registers, 12-bit digits starting at the highest bit in which the
//           row's keys differ, everything in one launch;
//   compact (long rows): a histogram pass over the top digit; a pass that
//           counts, per segment, the keys above the threshold bin and appends
//           the keys inside it to a candidate list; one workgroup per row that
//           finishes the selection on the candidates (and breaks ties by slot)
//           and turns per-segment counts into output offsets; an ordered
//           write pass -- three passes over the scores, five launches;
//   multipass (long rows whose candidate lists would not fit the workspace
//           budget): three histogram passes over the whole row, a counting
//           pass and an ordered write pass.
#include <algorithm>

#include "internal.hpp"
#include "tile.hpp"

namespace csa2 {

constexpr int kBins = 2048;
constexpr int kSeg = 8192;          // slots per workgroup in the streaming passes
constexpr int kThreads = 256;

struct RowState {
  uint32_t prefix;    // key bits fixed so far
  uint32_t need;      // slots still to take among keys matching prefix
  uint32_t k_eff;     // min(k, visible)
  uint32_t pad;
};

__device__ __forceinline__ uint32_t slot_key(const float* row, const int32_t* map_row, int64_t i) {
  uint32_t k = score_key(row[i]);
  if (map_row && map_row[i] < 0) k = 0u;
  return k;
}

__device__ __forceinline__ int digit_shift(int d) { return d == 0 ? 21 : (d == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask_above(int d) {
  return d == 0 ? 0u : (d == 1 ? 0xFFE00000u : 0xFFFFFC00u);
}

__global__ void __launch_bounds__(kThreads)
topk_init_kernel(uint32_t* __restrict__ hist, RowState* __restrict__ st) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[(int64_t)r * kBins + i] = 0u;
  if (threadIdx.x == 0) st[r] = RowState{0u, 0u, 0u, 0u};
}

template <int D>
__global__ void __launch_bounds__(kThreads)
topk_hist_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                 uint32_t* __restrict__ hist, const RowState* __restrict__ st) {
  __shared__ uint32_t h[kBins];
  const int r = blockIdx.y;
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
  __syncthreads();
  const RowState s = st ? st[r] : RowState{0u, 1u, 0u, 0u};
  const bool live = (D == 0) || s.need > 0;
  if (live) {
    const float* row = scores + (int64_t)r * stride;
    const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
    const uint32_t mask = digit_mask_above(D);
    const int shift = digit_shift(D);
    const int64_t b0 = (int64_t)blockIdx.x * kSeg;
    const int64_t b1 = min(N, b0 + kSeg);
    // kSeg = 8 x (256 threads x 4 slots): all eight 16-byte loads are issued first
    // (N is a multiple of 4, so a 4-slot group never straddles the row end)
    float4 v[8];
    int4 mp[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t i = b0 + (int64_t)q * kThreads * 4 + threadIdx.x * 4;
      v[q] = i < b1 ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      mp[q] = (map_row && i < b1) ? *reinterpret_cast<const int4*>(map_row + i) : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t i = b0 + (int64_t)q * kThreads * 4 + threadIdx.x * 4;
      if (i >= b1) continue;
      uint32_t k4[4] = {score_key(v[q].x), score_key(v[q].y), score_key(v[q].z), score_key(v[q].w)};
      int m4[4] = {mp[q].x, mp[q].y, mp[q].z, mp[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t k = m4[j] < 0 ? 0u : k4[j];
        if (k != 0u && (k & mask) == s.prefix) atomicAdd(&h[(k >> shift) & (kBins - 1)], 1u);
      }
    }
  }
  __syncthreads();
  if (live) {
    uint32_t* g = hist + (int64_t)r * kBins;
    for (int i = threadIdx.x; i < kBins; i += kThreads)
      if (h[i]) atomicAdd(&g[i], h[i]);
  }
}

// block-wide exclusive prefix sum of one value per thread (256 threads); the
// wave scans run on DPP row shifts and broadcasts, not LDS lane exchanges
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp /* >= 4 */, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  const uint32_t t0 = tmp[0], t1 = tmp[1], t2 = tmp[2], t3 = tmp[3];
  const uint32_t base = (wave > 0 ? t0 : 0u) + (wave > 1 ? t1 : 0u) + (wave > 2 ? t2 : 0u);
  total = t0 + t1 + t2 + t3;
  __syncthreads();
  return base + x - v;
}

// the same for N values per thread at once (one pair of barriers); tmp >= 4 N
template <int N>
__device__ __forceinline__ void block_exclusive_scan_n(const uint32_t (&v)[N], uint32_t (&excl)[N], uint32_t* tmp,
                                                       uint32_t (&total)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i] = wave_inclusive_scan(v[i]);
    if (lane == 63) tmp[4 * i + wave] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t t0 = tmp[4 * i], t1 = tmp[4 * i + 1], t2 = tmp[4 * i + 2], t3 = tmp[4 * i + 3];
    excl[i] = (wave > 0 ? t0 : 0u) + (wave > 1 ? t1 : 0u) + (wave > 2 ? t2 : 0u) + x[i] - v[i];
    total[i] = t0 + t1 + t2 + t3;
  }
  __syncthreads();
}

// Find the digit value holding the need-th largest remaining key.
template <int D>
__global__ void __launch_bounds__(kThreads)
topk_select_kernel(uint32_t* __restrict__ hist, RowState* __restrict__ st, int32_t k) {
  __shared__ uint32_t tmp[4];
  __shared__ uint32_t s_digit, s_above;
  const int r = blockIdx.x;
  uint32_t* g = hist + (int64_t)r * kBins;
  RowState s = st[r];
  // thread t owns bins [kBins-8t-8, kBins-8t) read from the top down
  uint32_t c[8];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int bin = kBins - 1 - (threadIdx.x * 8 + j);
    c[j] = g[bin];
    if (D == 0 && bin == 0) c[j] = 0u;      // key 0 = invisible
    local += c[j];
  }
  uint32_t total;
  uint32_t excl = block_exclusive_scan(local, tmp, total);
  uint32_t need = s.need;
  if (D == 0) {
    need = total < (uint32_t)k ? total : (uint32_t)k;      // k_eff = min(k, visible)
  }
  if (threadIdx.x == 0) { s_digit = 0xFFFFFFFFu; s_above = 0u; }
  __syncthreads();
  if (need > 0 && excl < need && need <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (acc < need && need <= acc + c[j]) {
        s_digit = (uint32_t)(kBins - 1 - (threadIdx.x * 8 + j));
        s_above = acc;
      }
      acc += c[j];
    }
  }
  __syncthreads();
  // clear the histogram for the next digit
#pragma unroll
  for (int j = 0; j < 8; ++j) g[kBins - 1 - (threadIdx.x * 8 + j)] = 0u;
  if (threadIdx.x == 0) {
    if (D == 0) s.k_eff = need;
    if (need == 0 || s_digit == 0xFFFFFFFFu) {
      s.need = 0u;
      s.prefix = 0xFFFFFFFFu;       // nothing to select
    } else {
      s.prefix |= s_digit << digit_shift(D);
      s.need = need - s_above;
    }
    st[r] = s;
  }
}

// per-segment counts of keys > tau and == tau
__global__ void __launch_bounds__(kThreads)
topk_count_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                  const RowState* __restrict__ st, uint32_t* __restrict__ seg_counts, int n_seg) {
  __shared__ uint32_t tmp[8];
  const int r = blockIdx.y;
  const RowState s = st[r];
  const uint32_t tau = s.prefix;
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int64_t b0 = (int64_t)blockIdx.x * kSeg;
  const int64_t b1 = min(N, b0 + kSeg);
  uint32_t gt = 0, eq = 0;
  if (s.k_eff > 0) {
    for (int64_t i = b0 + threadIdx.x; i < b1; i += kThreads) {
      uint32_t key = slot_key(row, map_row, i);
      gt += key > tau && key != 0u;
      eq += key == tau;
    }
  }
  // block reduce
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt += __shfl_xor(gt, o, 64);
    eq += __shfl_xor(eq, o, 64);
  }
  if (lane == 0) { tmp[wave] = gt; tmp[4 + wave] = eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* out = seg_counts + ((int64_t)r * n_seg + blockIdx.x) * 2;
    out[0] = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    out[1] = tmp[4] + tmp[5] + tmp[6] + tmp[7];
  }
}

// ordered write of the selected slots
__global__ void __launch_bounds__(kThreads)
topk_write_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                  const RowState* __restrict__ st, const uint32_t* __restrict__ seg_counts, int n_seg, int32_t k,
                  int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  __shared__ uint32_t tmp[8];
  __shared__ uint32_t s_off_gt, s_off_eq;
  const int r = blockIdx.y;
  const RowState s = st[r];
  const uint32_t tau = s.prefix;
  const uint32_t need_eq = s.need;
  const uint32_t k_eff = s.k_eff;
  int32_t* orow = idx_out + (int64_t)r * k;
  float* srow = score_out ? score_out + (int64_t)r * k : nullptr;

  // padding: the last segment's workgroup fills [k_eff, k)
  if (blockIdx.x == n_seg - 1) {
    for (int i = (int)k_eff + threadIdx.x; i < k; i += kThreads) {
      orow[i] = -1;
      if (srow) srow[i] = __builtin_nanf("");
    }
  }
  if (k_eff == 0) return;

  // offsets from earlier segments
  uint32_t a_gt = 0, a_eq = 0;
  const uint32_t* cnt = seg_counts + (int64_t)r * n_seg * 2;
  for (int sgi = threadIdx.x; sgi < blockIdx.x; sgi += kThreads) {
    a_gt += cnt[2 * sgi];
    a_eq += cnt[2 * sgi + 1];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a_gt += __shfl_xor(a_gt, o, 64);
    a_eq += __shfl_xor(a_eq, o, 64);
  }
  if (lane == 0) { tmp[wave] = a_gt; tmp[4 + wave] = a_eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_off_gt = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    s_off_eq = tmp[4] + tmp[5] + tmp[6] + tmp[7];
  }
  __syncthreads();
  uint32_t eq_seen = s_off_eq;                                      // equal keys before this point
  uint32_t out_pos = s_off_gt + min(s_off_eq, need_eq);             // output slots before this point

  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int64_t b0 = (int64_t)blockIdx.x * kSeg;
  const int64_t b1 = min(N, b0 + kSeg);
  __shared__ uint32_t tmp2[4];
  for (int64_t base = b0; base < b1; base += kThreads * 4) {
    // thread t owns slots [base + 4t, base + 4t + 4)
    uint32_t keys[4];
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t i = base + threadIdx.x * 4 + j;
      keys[j] = i < b1 ? slot_key(row, map_row, i) : 0u;
      n_gt += keys[j] > tau && keys[j] != 0u;
      n_eq += keys[j] == tau && keys[j] != 0u;
    }
    uint32_t tot_eq;
    uint32_t eq_before = block_exclusive_scan((uint32_t)n_eq, tmp2, tot_eq);
    // selected = gt plus eq whose global rank < need_eq
    uint32_t e0 = eq_seen + eq_before;
    int n_sel = n_gt;
    {
      uint32_t e = e0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (keys[j] == tau && keys[j] != 0u) { n_sel += e < need_eq; ++e; }
    }
    uint32_t tot_sel;
    uint32_t sel_before = block_exclusive_scan((uint32_t)n_sel, tmp2, tot_sel);
    uint32_t p = out_pos + sel_before;
    uint32_t e = e0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t i = base + threadIdx.x * 4 + j;
      bool take = false;
      if (keys[j] != 0u) {
        if (keys[j] > tau) take = true;
        else if (keys[j] == tau) { take = e < need_eq; ++e; }
      }
      if (take && p < k_eff) {
        orow[p] = map_row ? map_row[i] : (int32_t)i;
        if (srow) srow[p] = row[i];
        ++p;
      }
    }
    eq_seen += tot_eq;
    out_pos += tot_sel;
  }
}

// block-wide exclusive scan for 1024 threads (16 waves)
__device__ __forceinline__ uint32_t block_exclusive_scan_1024(uint32_t v, uint32_t* tmp /* >= 17 */,
                                                              uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < 16; ++w) { uint32_t t = tmp[w]; tmp[w] = acc; acc += t; }
    tmp[16] = acc;
  }
  __syncthreads();
  uint32_t res = tmp[wave] + x - v;
  total = tmp[16];
  __syncthreads();
  return res;
}

// Digit search over a 2048-bin histogram held in LDS by a 1024-thread block:
// the digit value holding the need-th largest key, and how many keys lie above it.
__device__ __forceinline__ void find_digit_1024(const uint32_t* h, uint32_t need, bool skip_bin0, uint32_t* tmp,
                                                uint32_t* s_digit, uint32_t* s_above, uint32_t& total) {
  const int t = threadIdx.x;
  const int b_hi = kBins - 1 - 2 * t, b_lo = kBins - 2 - 2 * t;
  uint32_t c_hi = h[b_hi];
  uint32_t c_lo = (skip_bin0 && b_lo == 0) ? 0u : h[b_lo];
  uint32_t excl = block_exclusive_scan_1024(c_hi + c_lo, tmp, total);
  if (t == 0) { *s_digit = 0xFFFFFFFFu; *s_above = 0u; }
  __syncthreads();
  if (need > 0) {
    if (excl < need && need <= excl + c_hi) { *s_digit = b_hi; *s_above = excl; }
    else if (excl + c_hi < need && need <= excl + c_hi + c_lo) { *s_digit = b_lo; *s_above = excl + c_hi; }
  }
  __syncthreads();
}

// ----------------------------------------------------------------------------
// small path: one 1024-thread workgroup per row, keys held in registers
// ----------------------------------------------------------------------------
constexpr int kSmallMax = 32768;
constexpr int kSmallThreads = 1024;
constexpr int kSmallBits = 12;
constexpr int kSmallBins = 1 << kSmallBits;


// Thread t owns the 4J consecutive slots [4J t, 4J t + 4J) of the row (4096 J
// >= N), with their index_map entries, in registers.  The k-th largest visible
// key tau is found by up to three radix digits of 12, 10 and 10 bits (from bit
// 31; the first histogram's total is the visible count), each in a histogram of
// its own (all three cleared up front): when the boundary bin of a digit holds
// exactly the keys still needed, the whole bin is taken and the later digits
// are skipped (tau = one below the bin, no ties to resolve) -- after the second
// digit this is the usual case.  The ordered write then needs one block scan of
// the threads' (above tau, equal to tau) counts, since thread order is slot
// order.  A second selection (k2 <= k, positions only) reuses the keys in
// registers: when k2 == k it is written by the same pass.
template <int J>
__global__ void __launch_bounds__(kSmallThreads)
topk_small_kernel(const float* __restrict__ scores, int N, int64_t stride, const int32_t* __restrict__ index_map,
                  int32_t k, int32_t* __restrict__ idx_out, float* __restrict__ score_out, int32_t k2,
                  int32_t* __restrict__ idx2_out) {
  constexpr int kHistWords = kSmallBins + 2 * 1024;     // digit 0 (12 bits), digits 1 and 2 (10 bits)
  __shared__ uint32_t hh[kHistWords];
  __shared__ uint32_t wt[16];
  __shared__ uint32_t wt2[2][16];
  __shared__ uint32_t s_res[3][3];                      // per digit: bin, keys above it, keys in it
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int s0 = 4 * J * tid;

  uint32_t key[J][4];
  int32_t pos[J][4];
  {
    float4 v[J];
    int4 mp[J];
    // every load unconditional (slots past N re-read the row's first four, N >= 4, and are masked after):
    // a load under a branch made the compiler wait for each before issuing the next
    if (map_row) {
#pragma unroll
      for (int it = 0; it < J; ++it) {
        const int sc = s0 + 4 * it < N ? s0 + 4 * it : 0;
        v[it] = *reinterpret_cast<const float4*>(row + sc);
        mp[it] = *reinterpret_cast<const int4*>(map_row + sc);
      }
    } else {
#pragma unroll
      for (int it = 0; it < J; ++it) {
        const int sc = s0 + 4 * it < N ? s0 + 4 * it : 0;
        v[it] = *reinterpret_cast<const float4*>(row + sc);
        mp[it] = make_int4(sc, sc + 1, sc + 2, sc + 3);
      }
    }
    // the histograms are cleared while the loads are in flight
    for (int i = tid; i < kHistWords; i += kSmallThreads) hh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < J; ++it) {
      const bool in = s0 + 4 * it < N;
      const float f[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
      const int32_t m4[4] = {mp[it].x, mp[it].y, mp[it].z, mp[it].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[it][j] = (!in || m4[j] < 0) ? 0u : score_key(f[j]);
        pos[it][j] = in ? m4[j] : -1;
        // the first selection's top digit, counted as each load lands
        if (key[it][j] != 0u) atomicAdd(&hh[key[it][j] >> 20], 1u);
      }
    }
  }

  // block scan whose wave totals go to one of two buffers, so that it needs a
  // single barrier (a buffer is reused only two digits later, past other barriers)
  auto scan1 = [&](uint32_t v, uint32_t* w, uint32_t& total) -> uint32_t {
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == 63) w[wave] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
      const uint32_t t = w[w2];
      base += w2 < wave ? t : 0u;
      tot += t;
    }
    total = tot;
    return base + inc - v;
  };

  // radix select of tau, the k_eff-th largest visible key (k_eff = min(kk, visible))
  auto select = [&](uint32_t kk, uint32_t& tau, uint32_t& need_eq, uint32_t& k_eff, bool first) {
    // the first selection finds its histograms cleared and the top digit's counted
    if (!first) {
      for (int i = tid; i < kHistWords; i += kSmallThreads) hh[i] = 0u;
      __syncthreads();
    }
    uint32_t need = 0, prefix = 0u;
    k_eff = 0;
    bool whole_bin = false;
#pragma unroll 1
    for (int d = 0; d < 3; ++d) {
      const int shift = d == 0 ? 20 : (d == 1 ? 10 : 0);
      const int hi = d == 0 ? 32 : (d == 1 ? 20 : 10);
      const uint32_t bmask = d == 0 ? 4095u : 1023u;
      const int nb = d == 0 ? 4096 : 1024;
      uint32_t* h = hh + (d == 0 ? 0 : kSmallBins + 1024 * (d - 1));
      if (d > 0 || !first) {
#pragma unroll
        for (int it = 0; it < J; ++it)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t x = key[it][j];
            if (x != 0u && (hi == 32 || (x >> hi) == (prefix >> hi))) atomicAdd(&h[(x >> shift) & bmask], 1u);
          }
      }
      __syncthreads();
      // bins walked from the top: 4 per thread at the first digit, 1 after
      const int per = d == 0 ? 4 : 1;
      uint32_t c[4] = {0u, 0u, 0u, 0u}, local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < per) {
          c[j] = h[nb - 1 - per * tid - j];
          local += c[j];
        }
      uint32_t total;
      const uint32_t excl = scan1(local, wt2[d & 1], total);
      if (d == 0) {
        k_eff = total < kk ? total : kk;     // total = visible keys
        need = k_eff;
      }
      if (need == 0u) break;
      if (excl < need && need <= excl + local) {
        uint32_t acc = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < per) {
            if (acc < need && need <= acc + c[j]) {
              s_res[d][0] = (uint32_t)(nb - 1 - per * tid - j);
              s_res[d][1] = acc;
              s_res[d][2] = c[j];
            }
            acc += c[j];
          }
      }
      __syncthreads();
      prefix |= s_res[d][0] << shift;
      need -= s_res[d][1];
      // every key of the boundary bin [prefix, prefix + 2^shift) is taken: tau
      // one below the bin selects exactly the keys above it and the bin
      if (need == s_res[d][2] && prefix != 0u) {
        whole_bin = true;
        break;
      }
    }
    tau = whole_bin ? prefix - 1u : prefix;
    need_eq = whole_bin ? 0u : need;
  };

  // ordered write: a slot's output index is (#keys > tau before it) + min(#keys == tau before it, need_eq);
  // orow2 (or null) takes the same positions
  auto write = [&](uint32_t tau, uint32_t need_eq, uint32_t k_eff, int32_t k_out, int32_t* orow, float* srow,
                   int32_t* orow2) {
    if (k_eff > 0) {
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int it = 0; it < J; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = key[it][j];
          cg += x != 0u && x > tau;
          ce += x != 0u && x == tau;
        }
      // both counts in one scan: each stays below 2^16 (N <= 32768)
      uint32_t tot;
      const uint32_t pre = block_scan_1024((cg << 16) | ce, wt, tot);
      uint32_t g = pre >> 16, e = pre & 0xFFFFu;
#pragma unroll
      for (int it = 0; it < J; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = key[it][j];
          const bool is_gt = x != 0u && x > tau;
          const bool is_eq = x != 0u && x == tau;
          const bool take = is_gt || (is_eq && e < need_eq);
          const uint32_t o = g + (is_gt ? min(e, need_eq) : e);
          g += is_gt ? 1u : 0u;
          e += is_eq ? 1u : 0u;
          if (take && o < k_eff) {
            orow[o] = pos[it][j];
            if (orow2) orow2[o] = pos[it][j];
            if (srow) srow[o] = key_score(x);
          }
        }
    }
    for (int i = (int)k_eff + tid; i < k_out; i += kSmallThreads) {
      orow[i] = -1;
      if (orow2) orow2[i] = -1;
      if (srow) srow[i] = __builtin_nanf("");
    }
  };

  uint32_t tau, need_eq, k_eff;
  select((uint32_t)k, tau, need_eq, k_eff, true);
  const bool same = idx2_out && k2 == k;
  write(tau, need_eq, k_eff, k, idx_out + (int64_t)r * k, score_out ? score_out + (int64_t)r * k : nullptr,
        same ? idx2_out + (int64_t)r * k2 : nullptr);
  if (idx2_out && !same) {
    __syncthreads();
    select((uint32_t)k2, tau, need_eq, k_eff, false);
    write(tau, need_eq, k_eff, k2, idx2_out + (int64_t)r * k2, nullptr, nullptr);
  }
}

// ----------------------------------------------------------------------------
// compact path (long rows)
// ----------------------------------------------------------------------------
constexpr int kTopBits = 12;                    // top digit: key bits 31..20
constexpr int kTopBins = 1 << kTopBits;
constexpr int kTopShift = 32 - kTopBits;

// histogram of the top 12 key bits of every visible slot (one 8192-slot segment per workgroup)
__global__ void __launch_bounds__(kThreads)
topk_top_hist_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                     uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kTopBins];
  const int r = blockIdx.y;
  for (int i = threadIdx.x; i < kTopBins; i += kThreads) h[i] = 0u;
  __syncthreads();
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int64_t b0 = (int64_t)blockIdx.x * kSeg;
  const int64_t b1 = min(N, b0 + kSeg);
  float4 v[8];
  int4 mp[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t i = b0 + (int64_t)q * kThreads * 4 + threadIdx.x * 4;
    v[q] = i < b1 ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    mp[q] = (map_row && i < b1) ? *reinterpret_cast<const int4*>(map_row + i) : make_int4(0, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t i = b0 + (int64_t)q * kThreads * 4 + threadIdx.x * 4;
    if (i >= b1) continue;
    const float f[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
    const int m4[4] = {mp[q].x, mp[q].y, mp[q].z, mp[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t k = m4[j] < 0 ? 0u : score_key(f[j]);
      if (k != 0u) atomicAdd(&h[k >> kTopShift], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = hist + (int64_t)r * kTopBins;
  for (int i = threadIdx.x; i < kTopBins; i += kThreads)
    if (h[i]) atomicAdd(&g[i], h[i]);
}
// The top digit b0 of the k-th largest key comes from the 12-bit histogram.
// Every visible key whose top digit is >= b0 is a candidate: keys above bin b0
// are all selected, keys inside it are resolved by the two lower digits.  Each
// segment writes its candidates (key, output position) in slot order into its
// own slot range, the segments are concatenated into one slot-ordered list per
// row, and one workgroup per row finishes the selection on that list -- about
// k plus one bin's worth of entries instead of N.  A second, smaller k2 can be
// selected from the same candidates (the top k2 lie inside the top k).

__global__ void __launch_bounds__(kThreads)
topk_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) p[i] = 0u;
}

// top digit b0 of the k-th largest visible key, and k_eff = min(k, visible), from a
// row's 12-bit top-digit histogram (256 threads; bin 0 holds only invisible keys)
__device__ __forceinline__ void derive_b0(const uint32_t* g, int32_t k, uint32_t* tmp, uint32_t& b0, uint32_t& k_eff) {
  __shared__ uint32_t s_digit;
  constexpr int kPer = kTopBins / kThreads;
  uint32_t c[kPer];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int bin = kTopBins - 1 - (threadIdx.x * kPer + j);
    c[j] = bin == 0 ? 0u : g[bin];
    local += c[j];
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(local, tmp, total);
  const uint32_t need = total < (uint32_t)k ? total : (uint32_t)k;
  if (threadIdx.x == 0) s_digit = 0xFFFFFFFFu;
  __syncthreads();
  if (need > 0 && excl < need && need <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (acc < need && need <= acc + c[j]) s_digit = (uint32_t)(kTopBins - 1 - (threadIdx.x * kPer + j));
      acc += c[j];
    }
  }
  __syncthreads();
  k_eff = need;
  b0 = s_digit;
  __syncthreads();
}

constexpr int kCompactBlock = kThreads * 32;     // slots per block step: thread t takes 32 consecutive slots

// per segment: the candidates (top digit >= b0) in slot order, written to the
// segment's own slot range of seg_key / seg_pos; their count to seg_cnt
__global__ void __launch_bounds__(kThreads)
topk_compact_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                    int32_t k, int seg, const uint32_t* __restrict__ hist0, uint32_t* __restrict__ seg_key,
                    int32_t* __restrict__ seg_pos, uint32_t* __restrict__ seg_cnt, int n_seg) {
  __shared__ uint32_t tmp[8];
  const int r = blockIdx.y;
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int64_t s0 = (int64_t)blockIdx.x * seg;
  const int64_t s1 = min(N, s0 + seg);
  uint32_t* okey = seg_key + (int64_t)r * N + s0;
  int32_t* opos = seg_pos + (int64_t)r * N + s0;
  // thread t takes 32 consecutive slots of each 8192-slot block; positions are
  // recomputed (or read from the map) only for the candidates
  auto load32 = [&](int64_t i0, uint32_t* keys) {
    float4 v[8];
    int4 mp[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t i = i0 + 4 * q;
      v[q] = i < s1 ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      mp[q] = (map_row && i < s1) ? *reinterpret_cast<const int4*>(map_row + i) : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = i0 + 4 * q < s1;
      const float f[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      const int32_t m4[4] = {mp[q].x, mp[q].y, mp[q].z, mp[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) keys[4 * q + j] = (!in || m4[j] < 0) ? 0u : score_key(f[j]);
    }
  };
  uint32_t keys[32];
  load32(s0 + (int64_t)threadIdx.x * 32, keys);      // in flight while b0 is derived
  uint32_t b0, k_eff;
  derive_b0(hist0 + (int64_t)r * kTopBins, k, tmp, b0, k_eff);
  uint32_t running = 0;
  if (k_eff > 0) {
    for (int64_t blk = s0; blk < s1; blk += kCompactBlock) {
      const int64_t i0 = blk + (int64_t)threadIdx.x * 32;
      if (blk != s0) load32(i0, keys);
      uint32_t sel = 0;                       // bit j: slot i0 + j is a candidate
#pragma unroll
      for (int j = 0; j < 32; ++j) sel |= (keys[j] != 0u && (keys[j] >> kTopShift) >= b0) ? (1u << j) : 0u;
      uint32_t total;
      uint32_t p = running + block_exclusive_scan((uint32_t)__popc(sel), tmp, total);
      while (sel) {
        const int j = __builtin_ctz(sel);
        sel &= sel - 1u;
        const int64_t i = i0 + j;
        okey[p] = keys[j];
        opos[p] = map_row ? map_row[i] : (int32_t)i;
        ++p;
      }
      running += total;
    }
  }
  if (threadIdx.x == 0) seg_cnt[(int64_t)r * n_seg + blockIdx.x] = running;
}

// concatenate the segments' candidate runs into one slot-ordered list per row
__global__ void __launch_bounds__(kThreads)
topk_flatten_kernel(int64_t N, int seg, const uint32_t* __restrict__ seg_key, const int32_t* __restrict__ seg_pos,
                    const uint32_t* __restrict__ seg_cnt, int n_seg, uint32_t* __restrict__ cand_key,
                    int32_t* __restrict__ cand_pos, uint32_t* __restrict__ cand_total) {
  __shared__ uint32_t red[4];
  const int r = blockIdx.y;
  const int si = blockIdx.x;
  const uint32_t* cnt = seg_cnt + (int64_t)r * n_seg;
  uint32_t part = 0;
  for (int i = threadIdx.x; i < si; i += kThreads) part += cnt[i];
  part = wave_sum_u32(part);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  const uint32_t base = red[0] + red[1] + red[2] + red[3];
  const uint32_t n = cnt[si];
  const int64_t src = (int64_t)r * N + (int64_t)si * seg;
  const int64_t dst = (int64_t)r * N + base;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
    cand_key[dst + i] = seg_key[src + i];
    cand_pos[dst + i] = seg_pos[src + i];
  }
  if (si == n_seg - 1 && threadIdx.x == 0) cand_total[r] = base + n;
}

// Finishing the selection(s) on a row's slot-ordered candidate list takes two
// kernels: one workgroup per row stages the keys in LDS (when they fit), finds
// tau and the number of ties to take for each selection, and counts, per chunk
// of 1024 list entries, the keys above and equal to tau; then many workgroups
// write the outputs chunk by chunk, each starting from the counts of the chunks
// before it.  Selection 0 takes k (idx_out [+ score_out]); selection 1, if
// present, k2 <= k (idx2_out).
constexpr int kFinishThreads = 1024;
constexpr int kFinishLds = 32768;
constexpr int kLowBins = 1024;                  // digits 1 and 2: key bits 19..10 and 9..0
constexpr int kChunk = 1024;                    // list entries per write chunk
constexpr int kWriteBlocks = 64;                // write workgroups per row (grid-stride over chunks)

struct SelState {
  uint32_t tau[2];
  uint32_t need_eq[2];
  uint32_t k_eff[2];
  uint32_t pad[2];
};

template <int NS, bool kLds>
__device__ __forceinline__ void select_passes(const uint32_t* keys, uint32_t C, uint32_t (*h)[kLowBins], uint32_t* wt,
                                              uint32_t (*s_res)[2], uint32_t* tau, uint32_t* need) {
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int d = 1; d <= 2; ++d) {
    const int shift = d == 1 ? 10 : 0;
    const int hi_shift = d == 1 ? kTopShift : 10;
    for (int i = tid; i < kLowBins; i += kFinishThreads) {
#pragma unroll
      for (int s = 0; s < NS; ++s) h[s][i] = 0u;
    }
    __syncthreads();
    uint32_t pfx[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) pfx[s] = tau[s] >> hi_shift;
    // 16-byte reads: entries [4 (u 1024 + t), +4) of each 16384-entry block
    for (uint32_t b = 0; b < C; b += 4u * 4u * kFinishThreads) {
      uint4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t v = b + 4u * (u * kFinishThreads + tid);
        kv[u] = v < C ? *reinterpret_cast<const uint4*>(keys + v) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t v = b + 4u * (u * kFinishThreads + tid);
        const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int s = 0; s < NS; ++s)
            if (v + j < C && (k4[j] >> hi_shift) == pfx[s]) atomicAdd(&h[s][(k4[j] >> shift) & (kLowBins - 1)], 1u);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      find_bin_1024<kLowBins>(h[s], need[s], wt, s_res[s]);
      __syncthreads();
      tau[s] |= s_res[s][0] << shift;
      need[s] -= s_res[s][1];
      __syncthreads();
    }
  }
}

template <int NS, bool kLds>
__device__ __forceinline__ void chunk_counts(const uint32_t* keys, uint32_t C, const uint32_t* tau,
                                             uint32_t* chunk_cnt /* [n_chunks][2 NS] of this row */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t n_chunks = (C + kChunk - 1) / kChunk;
  for (uint32_t c = wave; c < n_chunks; c += 16) {
    uint32_t cg[NS], ce[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) { cg[s] = 0u; ce[s] = 0u; }
    uint4 kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t v = c * kChunk + u * 256 + 4 * lane;
      kv[u] = v < C ? *reinterpret_cast<const uint4*>(keys + v) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t v = c * kChunk + u * 256 + 4 * lane;
      const uint32_t k4[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          cg[s] += v + j < C && k4[j] > tau[s];
          ce[s] += v + j < C && k4[j] == tau[s];
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t a = wave_sum_u32(cg[s]), b = wave_sum_u32(ce[s]);
      if (lane == 0) { chunk_cnt[c * 2 * NS + 2 * s] = a; chunk_cnt[c * 2 * NS + 2 * s + 1] = b; }
    }
  }
}

template <int NS>
__global__ void __launch_bounds__(kFinishThreads)
topk_select_cand_kernel(int64_t N, const uint32_t* __restrict__ hist0, const uint32_t* __restrict__ cand_key,
                        const uint32_t* __restrict__ cand_total, int32_t k, int32_t k2,
                        SelState* __restrict__ st, uint32_t* __restrict__ chunk_cnt) {
  __shared__ __attribute__((aligned(16))) uint32_t s_keys[kFinishLds];
  __shared__ uint32_t h[NS][kLowBins];
  __shared__ uint32_t wt[16];
  __shared__ uint32_t s_res[NS][2];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t* ck = cand_key + (int64_t)r * N;
  const uint32_t C = uniform_u32(cand_total[r]);
  const bool in_lds = C <= (uint32_t)kFinishLds;
  const int32_t kk_[2] = {k, NS == 2 ? k2 : 0};

  // top-digit histogram loads issued before the key staging
  constexpr int kPer = kTopBins / kFinishThreads;
  uint32_t c[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int bin = kTopBins - 1 - kPer * tid - j;
    c[j] = bin == 0 ? 0u : hist0[(int64_t)r * kTopBins + bin];
  }
  if (in_lds) {
    for (uint32_t b = 0; b < C; b += 4u * 4u * kFinishThreads) {
      uint4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t v = b + 4u * (u * kFinishThreads + tid);
        kv[u] = v < C ? *reinterpret_cast<const uint4*>(ck + v) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t v = b + 4u * (u * kFinishThreads + tid);
        if (v < C) *reinterpret_cast<uint4*>(s_keys + v) = kv[u];
      }
    }
  }
  // visible count and the top digit of each selection's k-th key
  uint32_t k_eff[NS], need[NS], tau[NS];
  {
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) local += c[j];
    uint32_t V;
    const uint32_t excl = block_scan_1024(local, wt, V);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      k_eff[s] = V < (uint32_t)kk_[s] ? V : (uint32_t)kk_[s];
      const uint32_t nd = k_eff[s];
      if (nd > 0 && excl < nd && nd <= excl + local) {
        uint32_t acc = excl;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          if (acc < nd && nd <= acc + c[j]) { s_res[s][0] = kTopBins - 1 - kPer * tid - j; s_res[s][1] = acc; }
          acc += c[j];
        }
      }
    }
  }
  __syncthreads();
  const bool live = k_eff[0] > 0;               // k_eff[1] > 0 exactly when k_eff[0] > 0
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    tau[s] = live ? s_res[s][0] << kTopShift : 0u;
    need[s] = live ? k_eff[s] - s_res[s][1] : 0u;
  }
  uint32_t* cc = chunk_cnt + (int64_t)r * ((N + kChunk - 1) / kChunk) * 2 * NS;
  if (live) {
    if (in_lds) {
      select_passes<NS, true>(s_keys, C, h, wt, s_res, tau, need);
      chunk_counts<NS, true>(s_keys, C, tau, cc);
    } else {
      select_passes<NS, false>(ck, C, h, wt, s_res, tau, need);
      chunk_counts<NS, false>(ck, C, tau, cc);
    }
  }
  if (tid == 0) {
    SelState o;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      o.tau[s] = s < NS ? tau[s] : 0u;
      o.need_eq[s] = s < NS ? need[s] : 0u;
      o.k_eff[s] = s < NS ? k_eff[s] : 0u;
    }
    o.pad[0] = o.pad[1] = 0u;
    st[r] = o;
  }
}

// write kernel: 256 threads, thread t holds list entries [4t, 4t+4) of a chunk
template <int NS>
__global__ void __launch_bounds__(kThreads)
topk_write_cand_kernel(int64_t N, const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos,
                       const uint32_t* __restrict__ cand_total, const SelState* __restrict__ st,
                       const uint32_t* __restrict__ chunk_cnt, int32_t k, int32_t* __restrict__ idx_out,
                       float* __restrict__ score_out, int32_t k2, int32_t* __restrict__ idx2_out) {
  __shared__ uint32_t tmp[8];
  __shared__ uint32_t red[2 * NS][4];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const SelState S = st[r];
  const uint32_t C = uniform_u32(cand_total[r]);
  const uint32_t n_chunks = (C + kChunk - 1) / kChunk;
  const int32_t kk_[2] = {k, NS == 2 ? k2 : 0};
  int32_t* orow[2] = {idx_out + (int64_t)r * k, NS == 2 ? idx2_out + (int64_t)r * k2 : nullptr};
  float* srow = score_out ? score_out + (int64_t)r * k : nullptr;
  if (blockIdx.x == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      for (int i = (int)S.k_eff[s] + tid; i < kk_[s]; i += kThreads) {
        orow[s][i] = -1;
        if (s == 0 && srow) srow[i] = __builtin_nanf("");
      }
  }
  if (S.k_eff[0] == 0) return;
  const uint32_t* cc = chunk_cnt + (int64_t)r * ((N + kChunk - 1) / kChunk) * 2 * NS;
  const uint32_t* ck = cand_key + (int64_t)r * N;
  const int32_t* cp = cand_pos + (int64_t)r * N;
  for (uint32_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    // counts of the chunks before this one
    uint32_t pre[2 * NS];
#pragma unroll
    for (int q = 0; q < 2 * NS; ++q) pre[q] = 0u;
    for (uint32_t i = tid; i < c; i += kThreads)
#pragma unroll
      for (int q = 0; q < 2 * NS; ++q) pre[q] += cc[i * 2 * NS + q];
#pragma unroll
    for (int q = 0; q < 2 * NS; ++q) {
      const uint32_t a = wave_sum_u32(pre[q]);
      if (lane == 0) red[q][wave] = a;
    }
    const uint32_t v0 = c * kChunk + 4 * tid;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
    int4 pv = make_int4(0, 0, 0, 0);
    if (v0 < C) {
      kv = *reinterpret_cast<const uint4*>(ck + v0);
      pv = *reinterpret_cast<const int4*>(cp + v0);
    }
    __syncthreads();
    const uint32_t k4[4] = {kv.x, kv.y, kv.z, kv.w};
    const int32_t p4[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t base_g = red[2 * s][0] + red[2 * s][1] + red[2 * s][2] + red[2 * s][3];
      const uint32_t base_e = red[2 * s + 1][0] + red[2 * s + 1][1] + red[2 * s + 1][2] + red[2 * s + 1][3];
      uint32_t ng = 0, ne = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ng += v0 + j < C && k4[j] > S.tau[s];
        ne += v0 + j < C && k4[j] == S.tau[s];
      }
      uint32_t tot;
      uint32_t g = base_g + block_exclusive_scan(ng, tmp, tot);
      uint32_t e = base_e + block_exclusive_scan(ne, tmp, tot);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = v0 + j < C;
        const bool is_gt = in && k4[j] > S.tau[s];
        const bool is_eq = in && k4[j] == S.tau[s];
        const bool take = is_gt || (is_eq && e < S.need_eq[s]);
        const uint32_t o = g + (is_gt ? min(e, S.need_eq[s]) : e);
        g += is_gt ? 1u : 0u;
        e += is_eq ? 1u : 0u;
        if (take && o < S.k_eff[s]) {
          orow[s][o] = p4[j];
          if (s == 0 && srow) srow[o] = key_score(k4[j]);
        }
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// streaming path of the Full scan + pool selection
//
// Before the scan, a strided sample bounds each row's k-th largest key from
// below (tau_s); the scan stores every visible key >= tau_s, block by block in
// position order, and the histogram of the candidates' digits
// min((key - tau_s) >> sh, 4095).  Two multi-workgroup passes finish both
// selections (k and k2 <= k), each workgroup owning a run of blocks:
//  - gather: each workgroup finds each selection's boundary bin b0 (the bin of
//    the k-th candidate) from the histogram, counts its candidates in higher
//    bins and appends those in bin b0 (typically a few dozen per row) to a
//    short list;
//  - finish (one workgroup per row): the k-th key tau exactly from the list,
//    the number of keys equal to tau to take, and every gather workgroup's
//    output base (keys above tau and ties at tau in the blocks before it);
//  - write: each workgroup writes its selected candidates in position order,
//    ties at tau to the lowest positions.
// The result does not depend on tau_s and needs no scores (the call may skip
// writing them).  When fewer than k candidates arrive (tau_s was above the k-th
// key), the row is rebuilt: each gather workgroup rescores its positions with
// the scan's tile arithmetic and stores every visible key in its blocks, with a
// histogram of their top 12 bits; the finish workgroup then selects by radix
// passes over the blocks.  When a boundary bin overflows its list (massive
// ties), the blocks already hold every candidate and the finish workgroup
// selects by radix passes over them.  (The passes are separate launches: a
// device-scope fence per workgroup, to let the last gather workgroup finish the
// row, costs more than a launch here, and so does resolving the row again in
// every write workgroup.)
// ----------------------------------------------------------------------------
constexpr int kStreamGroups = 32;        // gather / write workgroups per row (at most)
constexpr int kListCap = 4096;           // boundary-bin list entries per row and selection
constexpr int kSG = 256;                 // threads per gather / write workgroup

struct StreamBase {
  uint32_t gt[2];                        // keys > tau in the workgroups before this one
  uint32_t eq[2];                        // keys == tau in the workgroups before this one
};

// What a gather workgroup hands to its row's finishing workgroup inside the
// same launch (boundary-bin list entries, its counts above the boundary bins)
// goes through agent-scope atomic stores and loads: they reach and read the
// device's coherence point directly, so the hand-off needs no release fence,
// which on this multi-XCD part writes back the writer's whole L2.
__device__ __forceinline__ void put_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_agent(uint2* p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), ((uint64_t)v.y << 32) | v.x, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t get_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 get_agent(const uint2* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<uint2*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}

// the need-th largest of n keys (need in [1, n]); returns it and sets rank_gt
// to the number of keys above it.  256 threads; keys in LDS or global memory.
__device__ uint32_t kth_largest_256(const uint32_t* keys, uint32_t n, uint32_t need, uint32_t* h /* 4096 */,
                                    uint32_t* tmp /* 8 */, uint32_t* res /* 2 */, uint32_t& rank_gt) {
  const int tid = threadIdx.x;
  if (n <= (uint32_t)kSG) {
    // rank by counting: thread i holds key i
    const uint32_t mine = tid < (int)n ? keys[tid] : 0u;
    uint32_t gt = 0u, eq = 0u;
    for (uint32_t j = 0; j < n; ++j) {
      const uint32_t o = keys[j];
      gt += o > mine;
      eq += o == mine;
    }
    if (tid == 0) res[0] = 0u;
    __syncthreads();
    if (tid < (int)n && gt < need && need <= gt + eq) {
      res[0] = mine;
      res[1] = gt;
    }
    __syncthreads();
    const uint32_t tau = res[0];
    rank_gt = res[1];
    __syncthreads();
    return tau;
  }
  uint32_t prefix = 0u, above = 0u;
#pragma unroll 1
  for (int d = 0; d < 3; ++d) {
    const int shift = d == 0 ? 20 : (d == 1 ? 10 : 0);
    const int hi = d == 0 ? 32 : (d == 1 ? 20 : 10);
    const int nb = d == 0 ? 4096 : 1024;
    for (int i = tid; i < nb; i += kSG) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += kSG) {
      const uint32_t kx = keys[i];
      if (hi == 32 || (kx >> hi) == (prefix >> hi)) atomicAdd(&h[(kx >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // bins from the top, nb / 256 per thread
    const int per = nb / kSG;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) local += h[nb - 1 - per * tid - j];
    uint32_t total;
    const uint32_t excl = block_exclusive_scan(local, tmp, total);
    if (excl < need && need <= excl + local) {
      uint32_t acc = excl;
      for (int j = 0; j < per; ++j) {
        const uint32_t c = h[nb - 1 - per * tid - j];
        if (acc < need && need <= acc + c) {
          res[0] = (uint32_t)(nb - 1 - per * tid - j);
          res[1] = acc;
        }
        acc += c;
      }
    }
    __syncthreads();
    prefix |= res[0] << shift;
    need -= res[1];
    above += res[1];
    __syncthreads();
  }
  rank_gt = above;
  return prefix;
}

// The first 8 candidates of a block and its count, loaded together (one round
// trip for the common block of a few candidates); the entries beyond the count
// are ignored.  Later entries are read 8 at a time, also past the count (the
// candidate array carries 64 bytes of tail padding, so every read stays inside
// the workspace).
struct BlockHead {
  uint32_t c;
  uint4 e[4];                             // (key, position) pairs 0-7
};

// Holds a loaded value at this point.  Without it the compiler moves each load
// of a block head into the branch that first uses it (the entries are used
// only below the count), so a thread waits for one memory round trip per
// candidate instead of one per block.
__device__ __forceinline__ void keep_loaded(const uint4& v) {
  asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

__device__ __forceinline__ BlockHead load_head(const uint2* kp, const uint32_t* cnt, int64_t blk, int bsz) {
  BlockHead h;
  const uint4* b = reinterpret_cast<const uint4*>(kp + blk * bsz);
  h.c = cnt[blk];
#pragma unroll
  for (int u = 0; u < 4; ++u) h.e[u] = b[u];
#pragma unroll
  for (int u = 0; u < 4; ++u) keep_loaded(h.e[u]);
  return h;
}

// candidates of block blk (bsz positions) in position order, f(key, position); hd = its head
template <class F>
__device__ __forceinline__ void for_block(const BlockHead& hd, const uint2* kp, int64_t blk, int bsz, F&& f) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if ((uint32_t)(2 * u) < hd.c) f(hd.e[u].x, (int32_t)hd.e[u].y);
    if ((uint32_t)(2 * u + 1) < hd.c) f(hd.e[u].z, (int32_t)hd.e[u].w);
  }
  // the rest eight entries at a time, all four loads in flight together
  const uint4* b = reinterpret_cast<const uint4*>(kp + blk * bsz);
  for (uint32_t e = 8; e < hd.c; e += 8) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = b[e / 2 + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) keep_loaded(v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (e + 2 * u < hd.c) f(v[u].x, (int32_t)v[u].y);
      if (e + 2 * u + 1 < hd.c) f(v[u].z, (int32_t)v[u].w);
    }
  }
}

// C = the row's candidate count, each selection's k_eff, boundary bin b0, the
// candidates above it (above) and in it (cb0); rebuild: fewer than k
// candidates (tau_s above the k-th key); overflow: a boundary bin holds more
// than a list takes.  256 threads, bins walked from the top.
struct RowBins {
  uint32_t C, k_eff[2], b0[2], above[2], cb0[2];
  bool rebuild, overflow;
};

__device__ __forceinline__ void bins_from_top(const uint32_t* hr, const uint32_t* need, uint32_t* tmp, uint32_t* s_b,
                                              uint32_t& total) {
  const int tid = threadIdx.x;
  constexpr int kPer = kStreamBins / kSG;
  static_assert(kPer == 16, "four 16-byte loads per thread");
  // thread tid's bins 4095 - 16 tid - j (j < 16): one contiguous 64-byte run, loaded as four vectors
  const uint4* h4 = reinterpret_cast<const uint4*>(hr + (kStreamBins - kPer * (tid + 1)));
  const uint4 v0 = h4[0], v1 = h4[1], v2 = h4[2], v3 = h4[3];
  const uint32_t c[kPer] = {v3.w, v3.z, v3.y, v3.x, v2.w, v2.z, v2.y, v2.x,
                            v1.w, v1.z, v1.y, v1.x, v0.w, v0.z, v0.y, v0.x};
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) local += c[j];
  const uint32_t excl = block_exclusive_scan(local, tmp, total);
  if (tid == 0)
    for (int i = 0; i < 6; ++i) s_b[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint32_t nd = min(need[s], total);
    if (nd > 0u && excl < nd && nd <= excl + local) {
      uint32_t acc = excl;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (acc < nd && nd <= acc + c[j]) {
          s_b[3 * s] = (uint32_t)(kStreamBins - 1 - kPer * tid - j);
          s_b[3 * s + 1] = acc;
          s_b[3 * s + 2] = c[j];
        }
        acc += c[j];
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ RowBins row_bins(const uint32_t* hr, uint32_t tau_s, int32_t k, int32_t k2, uint32_t* tmp,
                                            uint32_t* s_b /* 6 */) {
  const uint32_t kk[2] = {(uint32_t)k, (uint32_t)k2};
  RowBins rb;
  bins_from_top(hr, kk, tmp, s_b, rb.C);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    rb.k_eff[s] = tau_s == 0u ? min(kk[s], rb.C) : kk[s];
    rb.b0[s] = s_b[3 * s];
    rb.above[s] = s_b[3 * s + 1];
    rb.cb0[s] = s_b[3 * s + 2];
  }
  __syncthreads();
  rb.rebuild = tau_s != 0u && rb.C < kk[0];
  rb.overflow = !rb.rebuild && rb.k_eff[0] > 0u &&
                (rb.cb0[0] > (uint32_t)kListCap || rb.cb0[1] > (uint32_t)kListCap);
  return rb;
}

// Rebuild of a row whose threshold missed: the workgroup's blocks get every
// visible key of their positions (scored as in the scan: wave w takes blocks
// blk0 + w, blk0 + w + 4, ..., each block's tiles in order), and hist_abs the
// top 12 bits of those keys.
__device__ void rebuild_blocks(const uint8_t* q_idx, const uint8_t* k_idx, int64_t T, int r, const int32_t* row_seq,
                               const int64_t* row_limit, int64_t blk0, int64_t blk1, int bsz, uint2* kp, uint32_t* cn,
                               uint32_t* hist_abs, uint32_t* h /* 4096, LDS */, const PageMap& pm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kn = lane & 15, part = 16 * (lane >> 4);
  for (int i = tid; i < kStreamBins; i += kSG) h[i] = 0u;
  __syncthreads();
  const int seq = row_seq ? row_seq[r] : r;
  const int64_t limit = row_limit ? row_limit[r] : T - 1;
  f16x8 a[2];
  query_operands(q_idx + (int64_t)r * kIndexDim, lane, a);
  for (int64_t blk = blk0 + wave; blk < blk1; blk += 4) {
    uint32_t at = 0;
    for (int t = 0; t < bsz / kTile; t += 4) {
      i32x8 kb[4];
      bool ok[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t p0 = blk * bsz + kTile * (t + i);
        const int64_t row0 = p0 < T ? phys_row(pm, seq, T, p0) : -1;
        uint4 v[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int64_t p = p0 + 16 * hh + kn;
          ok[i][hh] = row0 >= 0 && p < T && p <= limit;
          v[hh] = ok[i][hh] ? load_key_part(k_idx + (row0 + 16 * hh + kn) * kIndexDim + part) : make_uint4(0, 0, 0, 0);
        }
        kb[i] = tile_pair(v[0], v[1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 sc = mfma_score(a, kb[i]);
        const float sv[2] = {sc.x, sc.y};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t key = (lane < 16 && ok[i][hh]) ? score_key(sv[hh]) : 0u;
          const bool c = key != 0u;
          const uint64_t m = __ballot(c);
          if (c) {
            kp[blk * bsz + at + lanes_below(m)] =
                make_uint2(key, (uint32_t)(blk * bsz + kTile * (t + i) + 16 * hh + kn));
            atomicAdd(&h[key >> 20], 1u);
          }
          at += (uint32_t)__popcll(m);
        }
      }
    }
    if (lane == 0) cn[blk] = at;
  }
  __syncthreads();
  for (int i = tid; i < kStreamBins; i += kSG)
    if (h[i]) atomicAdd(&hist_abs[i], h[i]);
}

// The candidate histogram of each row when the query-block scan produced the
// candidates (32 rows' 4,096-bin histograms do not fit one workgroup's LDS):
// one workgroup per row counts the digits of its blocks' candidates in LDS
// and stores the row's bins.
__global__ void __launch_bounds__(kSG)
stream_hist_kernel(int64_t T, int64_t nbk, int bsz, const StreamRow* __restrict__ rows, uint32_t* __restrict__ hist,
                   const uint2* __restrict__ cand, const uint32_t* __restrict__ cand_cnt) {
  __shared__ uint32_t h[kStreamBins];
  const int r = blockIdx.x, tid = threadIdx.x;
  const uint32_t tau_s = rows[r].tau_s, sh = rows[r].sh;
  const uint2* kp = cand + (int64_t)r * T;
  const uint32_t* cn = cand_cnt + (int64_t)r * nbk;
  for (int i = tid; i < kStreamBins; i += kSG) h[i] = 0u;
  __syncthreads();
  for (int64_t blk = tid; blk < nbk; blk += kSG)
    for_block(load_head(kp, cn, blk, bsz), kp, blk, bsz, [&](uint32_t kx, int32_t) {
      atomicAdd(&h[min((kx - tau_s) >> sh, (uint32_t)(kStreamBins - 1))], 1u);
    });
  __syncthreads();
  uint32_t* hr = hist + (int64_t)r * kStreamHistWords;
  for (int i = tid; i < kStreamBins; i += kSG) hr[i] = h[i];
}

// the need-th largest key among a row's candidate blocks that pass `keep`,
// starting from a known prefix: radix digits of the bits below bit `hi`
// (11 bits and then 10 at a time), prefix bits at and above `hi` must match.
// Returns tau; need becomes the number of keys equal to tau to take.
template <class Keep>
__device__ uint32_t select_in_blocks(const uint2* kp, const uint32_t* cn, int64_t nbk, int bsz, Keep keep, int hi,
                                     uint32_t prefix, uint32_t& need, uint32_t* h /* 2048 */, uint32_t* tmp,
                                     uint32_t* res) {
  const int tid = threadIdx.x;
#pragma unroll 1
  while (hi > 0) {
    const int width = hi > 10 ? (hi >= 21 ? 11 : hi - 10) : hi;
    const int shift = hi - width;
    const uint32_t mask = (1u << width) - 1u;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += kSG) h[i] = 0u;
    __syncthreads();
    for (int64_t blk = tid; blk < nbk; blk += kSG) {
      const BlockHead hd = load_head(kp, cn, blk, bsz);
      for_block(hd, kp, blk, bsz, [&](uint32_t kx, int32_t) {
        if (keep(kx) && (hi >= 32 || (kx >> hi) == (prefix >> hi))) atomicAdd(&h[(kx >> shift) & mask], 1u);
      });
    }
    __syncthreads();
    // bins from the top, nb / 256 (at least 1) per thread
    const int per = nb >= kSG ? nb / kSG : 1;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - per * tid - j;
      local += bin >= 0 ? h[bin] : 0u;
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan(local, tmp, total);
    if (excl < need && need <= excl + local) {
      uint32_t acc = excl;
      for (int j = 0; j < per; ++j) {
        const int bin = nb - 1 - per * tid - j;
        const uint32_t c = bin >= 0 ? h[bin] : 0u;
        if (acc < need && need <= acc + c) {
          res[0] = (uint32_t)bin;
          res[1] = acc;
        }
        acc += c;
      }
    }
    __syncthreads();
    prefix |= res[0] << shift;
    need -= res[1];
    hi = shift;
    __syncthreads();
  }
  return prefix;
}

// finish of row r, by the row's last gather workgroup.  From the short lists:
// each selection's k-th key tau, the ties at tau it takes, and for every gather
// workgroup the keys above tau and equal to tau in the blocks before it.  In a
// rebuilt or overflowing row, the k-th keys by radix passes over the blocks and
// the per-workgroup counts by a pass over them.
struct FinishLds {
  uint32_t* tmp;     // 8
  uint32_t* s_b;     // 6
  uint32_t* res;     // 2
  uint32_t* h;       // kStreamBins
  uint32_t* s_lk;    // kListCap, 16-byte aligned
  uint32_t* s_gt;    // kStreamGroups
  uint32_t* s_eq;    // kStreamGroups
  uint32_t* res2;    // 4
};

__device__ void finish_row(int r, int R, int64_t T, int64_t nbk, int bpw, int bsz, int G, StreamRow* __restrict__ rows,
                           const uint32_t* __restrict__ hist, const uint32_t* __restrict__ above_out,
                           const uint2* __restrict__ list, const uint2* __restrict__ cand,
                           const uint32_t* __restrict__ cand_cnt, StreamBase* __restrict__ base_out, int32_t k,
                           int32_t k2, const RowBins& rb, const FinishLds& lds) {
  uint32_t* tmp = lds.tmp;
  uint32_t* s_b = lds.s_b;
  uint32_t* res = lds.res;
  uint32_t* h = lds.h;
  uint32_t* s_lk = lds.s_lk;
  uint32_t* s_gt = lds.s_gt;
  uint32_t* s_eq = lds.s_eq;
  uint32_t* res2 = lds.res2;
  const int tid = threadIdx.x;
  struct {
    uint32_t tau_s, sh, n_list[2];
  } st;
  st.tau_s = rows[r].tau_s;
  st.sh = rows[r].sh;
  st.n_list[0] = get_agent(&rows[r].n_list[0]);
  st.n_list[1] = get_agent(&rows[r].n_list[1]);
  const uint32_t* hr = hist + (int64_t)r * kStreamHistWords;
  const uint2* kp = cand + (int64_t)r * T;
  const uint32_t* cn = cand_cnt + (int64_t)r * nbk;
  // entry tid of each list and workgroup tid's gather counts
  uint2 le0[2];
  uint32_t ab0[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    le0[s] = get_agent(&list[((int64_t)s * R + r) * kListCap + tid]);
    ab0[s] = tid < G ? get_agent(&above_out[((int64_t)r * G + tid) * 2 + s]) : 0u;
  }
  StreamBase* bo = base_out + (int64_t)r * G;
  const uint32_t kk[2] = {(uint32_t)k, (uint32_t)k2};
  uint32_t tau[2] = {0u, 0u}, need_eq[2] = {0u, 0u}, k_eff[2] = {rb.k_eff[0], rb.k_eff[1]};
  const uint32_t mode = rb.rebuild ? 1u : (rb.overflow ? 2u : 0u);
  if (mode == 0u && rb.k_eff[0] == 0u) {
    for (int i = tid; i < G; i += kSG) bo[i] = StreamBase{{0u, 0u}, {0u, 0u}};
  } else if (mode == 0u && st.n_list[0] <= (uint32_t)kSG && st.n_list[1] <= (uint32_t)kSG) {
    // both short lists at once (the usual case): thread i holds entry i of each,
    // ranks it by counting, and the workgroup counts follow in the same pass
    uint32_t* lk1 = s_lk + kSG;
    uint32_t* gts = s_gt;                         // [2][kStreamGroups] in s_gt / s_eq pairs below
    // entries past a list's end are 0, which no visible key equals or falls below
    s_lk[tid] = tid < (int)st.n_list[0] ? le0[0].x : 0u;
    lk1[tid] = tid < (int)st.n_list[1] ? le0[1].x : 0u;
    for (int i = tid; i < kStreamGroups; i += kSG) { s_gt[i] = 0u; s_eq[i] = 0u; h[i] = 0u; h[kStreamGroups + i] = 0u; }
    if (tid < 4) res2[tid] = 0u;
    __syncthreads();
    {
      // both lists in one pass, four entries per LDS read and several reads in flight
      const uint4* l0 = reinterpret_cast<const uint4*>(s_lk);
      const uint4* l1 = reinterpret_cast<const uint4*>(lk1);
      const uint32_t n4 = (max(st.n_list[0], st.n_list[1]) + 3u) >> 2;
      const uint32_t m0 = le0[0].x, m1 = le0[1].x;
      uint32_t gt[2] = {0u, 0u}, eq[2] = {0u, 0u};
#pragma unroll 4
      for (uint32_t j = 0; j < n4; ++j) {
        const uint4 a = l0[j], b = l1[j];
        gt[0] += (uint32_t)(a.x > m0) + (uint32_t)(a.y > m0) + (uint32_t)(a.z > m0) + (uint32_t)(a.w > m0);
        eq[0] += (uint32_t)(a.x == m0) + (uint32_t)(a.y == m0) + (uint32_t)(a.z == m0) + (uint32_t)(a.w == m0);
        gt[1] += (uint32_t)(b.x > m1) + (uint32_t)(b.y > m1) + (uint32_t)(b.z > m1) + (uint32_t)(b.w > m1);
        eq[1] += (uint32_t)(b.x == m1) + (uint32_t)(b.y == m1) + (uint32_t)(b.z == m1) + (uint32_t)(b.w == m1);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t n = st.n_list[s], need = rb.k_eff[s] - rb.above[s];
        if (tid < (int)n && gt[s] < need && need <= gt[s] + eq[s]) {
          res2[2 * s] = le0[s].x;
          res2[2 * s + 1] = gt[s];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      tau[s] = res2[2 * s];
      need_eq[s] = rb.k_eff[s] - rb.above[s] - res2[2 * s + 1];
      if (tid < (int)st.n_list[s]) {
        const uint32_t wg = (uint32_t)(((int64_t)(int32_t)le0[s].y / bsz) / bpw);
        uint32_t* cg = s == 0 ? s_gt : h;
        uint32_t* ce = s == 0 ? s_eq : h + kStreamGroups;
        if (le0[s].x > tau[s]) atomicAdd(&cg[wg], 1u);
        else if (le0[s].x == tau[s]) atomicAdd(&ce[wg], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // G <= 64: one wave scans the workgroups' counts of both selections
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t* cg = s == 0 ? s_gt : h;
        const uint32_t* ce = s == 0 ? s_eq : h + kStreamGroups;
        const uint32_t gtc = tid < G ? cg[tid] + ab0[s] : 0u;
        const uint32_t eqc = tid < G ? ce[tid] : 0u;
        const uint32_t gi = wave_inclusive_scan(gtc) - gtc, ei = wave_inclusive_scan(eqc) - eqc;
        if (tid < G) {
          bo[tid].gt[s] = gi;
          bo[tid].eq[s] = ei;
        }
      }
    }
    (void)gts;
  } else if (mode == 0u) {
#pragma unroll 1
    for (int s = 0; s < 2; ++s) {
      const uint32_t n = st.n_list[s];
      const uint2* ls = list + ((int64_t)s * R + r) * kListCap;
      for (uint32_t i = tid; i < n; i += kSG) s_lk[i] = i == (uint32_t)tid ? le0[s].x : get_agent(&ls[i]).x;
      for (int i = tid; i < G; i += kSG) { s_gt[i] = 0u; s_eq[i] = 0u; }
      __syncthreads();
      const uint32_t need = rb.k_eff[s] - rb.above[s];
      uint32_t gt_in_list;
      tau[s] = kth_largest_256(s_lk, n, need, h, tmp, res, gt_in_list);
      need_eq[s] = need - gt_in_list;
      for (uint32_t i = tid; i < n; i += kSG) {
        const int32_t p = (int32_t)(i == (uint32_t)tid ? le0[s].y : get_agent(&ls[i]).y);
        const uint32_t wg = (uint32_t)(((int64_t)p / bsz) / bpw);
        if (s_lk[i] > tau[s]) atomicAdd(&s_gt[wg], 1u);
        else if (s_lk[i] == tau[s]) atomicAdd(&s_eq[wg], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // G <= 64: one wave scans the workgroups' counts
        const uint32_t gtc = tid < G ? s_gt[tid] + ab0[s] : 0u;
        const uint32_t eqc = tid < G ? s_eq[tid] : 0u;
        const uint32_t gi = wave_inclusive_scan(gtc) - gtc, ei = wave_inclusive_scan(eqc) - eqc;
        if (tid < G) {
          bo[tid].gt[s] = gi;
          bo[tid].eq[s] = ei;
        }
      }
      __syncthreads();
    }
  } else {
    uint32_t b0[2], above[2];
    if (mode == 1u) {
      // every visible key is in the blocks; the second histogram holds their top 12 bits
      uint32_t V;
      bins_from_top(hr + kStreamBins, kk, tmp, s_b, V);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        k_eff[s] = min(kk[s], V);
        b0[s] = s_b[3 * s];
        above[s] = s_b[3 * s + 1];
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        b0[s] = rb.b0[s];
        above[s] = rb.above[s];
      }
    }
    if (k_eff[0] == 0u) {
      for (int i = tid; i < G; i += kSG) bo[i] = StreamBase{{0u, 0u}, {0u, 0u}};
    } else {
      const uint32_t tau_s = st.tau_s, sh = st.sh;
#pragma unroll 1
      for (int s = 0; s < 2; ++s) {
        uint32_t need = k_eff[s] - above[s];
        const uint32_t bs = b0[s];
        if (mode == 1u)
          tau[s] = select_in_blocks(kp, cn, nbk, bsz, [](uint32_t) { return true; }, 20, bs << 20, need, h, tmp, res);
        else
          tau[s] = select_in_blocks(
              kp, cn, nbk, bsz, [=](uint32_t kx) { return min((kx - tau_s) >> sh, (uint32_t)(kStreamBins - 1)) == bs; },
              32, 0u, need, h, tmp, res);
        need_eq[s] = need;
      }
      // keys > tau and == tau in each gather workgroup's blocks, then the bases
#pragma unroll 1
      for (int s = 0; s < 2; ++s) {
        for (int i = tid; i < G; i += kSG) { s_gt[i] = 0u; s_eq[i] = 0u; }
        __syncthreads();
        for (int64_t blk = tid; blk < nbk; blk += kSG) {
          uint32_t gt = 0u, eq = 0u;
          for_block(load_head(kp, cn, blk, bsz), kp, blk, bsz, [&](uint32_t kx, int32_t) {
            gt += kx > tau[s];
            eq += kx == tau[s];
          });
          if (gt) atomicAdd(&s_gt[blk / bpw], gt);
          if (eq) atomicAdd(&s_eq[blk / bpw], eq);
        }
        __syncthreads();
        if (tid < 64) {
          const uint32_t gtc = tid < G ? s_gt[tid] : 0u;
          const uint32_t eqc = tid < G ? s_eq[tid] : 0u;
          const uint32_t gi = wave_inclusive_scan(gtc) - gtc, ei = wave_inclusive_scan(eqc) - eqc;
          if (tid < G) {
            bo[tid].gt[s] = gi;
            bo[tid].eq[s] = ei;
          }
        }
        __syncthreads();
      }
    }
  }
  if (tid == 0) {
    StreamRow* o = &rows[r];
    o->mode = mode;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      o->tau[s] = tau[s];
      o->need_eq[s] = need_eq[s];
      o->k_eff[s] = k_eff[s];
    }
  }
}

// the gather pass over blocks [blk0, blk1) of row r: each boundary bin's
// entries appended to its list, and the workgroup's counts above the boundary
// bins, both handed to the finishing workgroup with agent-scope stores
__device__ __forceinline__ void gather_blocks(StreamRow* rows, int r, int R, int G, int g, int64_t blk0, int64_t blk1,
                                              int bsz, const uint2* kp, const uint32_t* cn, const BlockHead& hd0,
                                              uint32_t tau_s, uint32_t sh, const RowBins& rb, uint2* list,
                                              uint32_t* above_out, uint32_t* tmp) {
  const int tid = threadIdx.x;
  uint32_t ab[2] = {0u, 0u};
  for (int64_t blk = blk0 + tid; blk < blk1; blk += kSG) {
    const BlockHead hd = blk == blk0 + tid ? hd0 : load_head(kp, cn, blk, bsz);
    for_block(hd, kp, blk, bsz, [&](uint32_t kx, int32_t p) {
      const uint32_t d = min((kx - tau_s) >> sh, (uint32_t)(kStreamBins - 1));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (d > rb.b0[s]) ++ab[s];
        if (d == rb.b0[s]) {
          const uint32_t i = atomicAdd(&rows[r].n_list[s], 1u);
          put_agent(&list[((int64_t)s * R + r) * kListCap + i], make_uint2(kx, (uint32_t)p));
        }
      }
    });
  }
  {
    uint32_t ex[2], tot[2];
    block_exclusive_scan_n<2>(ab, ex, tmp, tot);
    if (tid == 0) {
      put_agent(&above_out[((int64_t)r * G + g) * 2], tot[0]);
      put_agent(&above_out[((int64_t)r * G + g) * 2 + 1], tot[1]);
    }
  }
}

// gather: per workgroup, the candidates above each boundary bin in its blocks,
// and the candidates inside the boundary bin appended to the row's short list;
// in a row to rebuild, the rebuild of its blocks instead.  The row's last
// workgroup to arrive (a ticket in the row's state, cleared by the threshold
// kernel) then finishes the row.
__global__ void __launch_bounds__(kSG)
stream_gather_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx, int64_t T,
                     const int32_t* __restrict__ row_seq, const int64_t* __restrict__ row_limit, int64_t nbk, int bpw,
                     int bsz, StreamRow* __restrict__ rows, uint32_t* __restrict__ hist, uint2* __restrict__ cand,
                     uint32_t* __restrict__ cand_cnt, uint32_t* __restrict__ above_out, uint2* __restrict__ list,
                     StreamBase* __restrict__ base_out, int32_t k, int32_t k2, PageMap pm) {
  __shared__ uint32_t tmp[8];
  __shared__ uint32_t s_b[6];
  __shared__ uint32_t h[kStreamBins];
  __shared__ uint32_t res[2];
  __shared__ __align__(16) uint32_t s_lk[kListCap];
  __shared__ uint32_t s_gt[kStreamGroups], s_eq[kStreamGroups];
  __shared__ uint32_t res2[4];
  __shared__ uint32_t s_last;
  const int r = blockIdx.y, g = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
  const int R = gridDim.y;
  const uint32_t tau_s = rows[r].tau_s, sh = rows[r].sh;
  uint2* kp = cand + (int64_t)r * T;
  uint32_t* cn = cand_cnt + (int64_t)r * nbk;
  uint32_t* hr = hist + (int64_t)r * kStreamHistWords;
  // the first block's head is loaded with the histogram
  const int64_t blk0 = (int64_t)g * bpw, blk1 = min(nbk, blk0 + bpw);
  BlockHead hd0 = {};
  if (blk0 + tid < blk1) hd0 = load_head(kp, cn, blk0 + tid, bsz);
  const RowBins rb = row_bins(hr, tau_s, k, k2, tmp, s_b);
  if (rb.rebuild) {
    rebuild_blocks(q_idx, k_idx, T, r, row_seq, row_limit, blk0, blk1, bsz, kp, cn, hr + kStreamBins, h, pm);
    // the rebuilt blocks and counts are plain stores: publish them (rare path)
    __threadfence();
  } else if (!rb.overflow && rb.k_eff[0] != 0u) {
    gather_blocks(rows, r, R, G, g, blk0, blk1, bsz, kp, cn, hd0, tau_s, sh, rb, list, above_out, tmp);
  }
  // every thread's hand-off stores have completed before the ticket is taken
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&rows[r].ticket, 1u) == (uint32_t)(G - 1) ? 1u : 0u;
  __syncthreads();
  if (s_last == 0u) return;
  if (rb.rebuild) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const FinishLds lds{tmp, s_b, res, h, s_lk, s_gt, s_eq, res2};
  finish_row(r, R, T, nbk, bpw, bsz, G, rows, hist, above_out, list, cand, cand_cnt, base_out, k, k2, rb, lds);
}


// ordered write: each workgroup's blocks, thread t taking a contiguous run of them
__global__ void __launch_bounds__(kSG)
stream_write_kernel(int64_t T, int64_t nbk, int bpw, int bsz, const StreamRow* __restrict__ rows,
                    const StreamBase* __restrict__ base, const uint2* __restrict__ cand,
                    const uint32_t* __restrict__ cand_cnt, int32_t k, int32_t k2, int32_t* __restrict__ idx_out,
                    float* __restrict__ score_out, int32_t* __restrict__ idx2_out) {
  __shared__ uint32_t tmp[16];
  const int r = blockIdx.y, g = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
  const uint2* kp = cand + (int64_t)r * T;
  const uint32_t* cn = cand_cnt + (int64_t)r * nbk;
  const int64_t blk0 = (int64_t)g * bpw, blk1 = min(nbk, blk0 + bpw);
  const int64_t per = (blk1 - blk0 + kSG - 1) / kSG;
  const int64_t my0 = min(blk1, blk0 + tid * per), my1 = min(blk1, my0 + per);
  BlockHead hd0 = {};
  if (my0 < my1) hd0 = load_head(kp, cn, my0, bsz);
  const StreamRow st = rows[r];
  const StreamBase bs = base[(int64_t)r * G + g];
  const uint32_t kk[2] = {(uint32_t)k, (uint32_t)k2};
  int32_t* orow[2] = {idx_out + (int64_t)r * k, idx2_out + (int64_t)r * k2};
  float* srow = score_out ? score_out + (int64_t)r * k : nullptr;
  if (g == 0) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      for (uint32_t i = st.k_eff[s] + tid; i < kk[s]; i += kSG) {
        orow[s][i] = -1;
        if (s == 0 && srow) srow[i] = __builtin_nanf("");
      }
  }
  if (st.k_eff[0] == 0u) return;
  uint32_t gt[2] = {0u, 0u}, eq[2] = {0u, 0u};
  for (int64_t blk = my0; blk < my1; ++blk)
    for_block(blk == my0 ? hd0 : load_head(kp, cn, blk, bsz), kp, blk, bsz, [&](uint32_t kx, int32_t) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        gt[s] += kx > st.tau[s];
        eq[s] += kx == st.tau[s];
      }
    });
  uint32_t gs[2], es[2];
  {
    const uint32_t v[4] = {gt[0], eq[0], gt[1], eq[1]};
    uint32_t ex[4], tot[4];
    block_exclusive_scan_n<4>(v, ex, tmp, tot);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      gs[s] = bs.gt[s] + ex[2 * s];
      es[s] = bs.eq[s] + ex[2 * s + 1];
    }
  }
  for (int64_t blk = my0; blk < my1; ++blk)
    for_block(blk == my0 ? hd0 : load_head(kp, cn, blk, bsz), kp, blk, bsz, [&](uint32_t kx, int32_t p) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bool is_gt = kx > st.tau[s], is_eq = kx == st.tau[s];
        const bool take = is_gt || (is_eq && es[s] < st.need_eq[s]);
        const uint32_t o = gs[s] + (is_gt ? min(es[s], st.need_eq[s]) : es[s]);
        if (take && o < st.k_eff[s]) {
          orow[s][o] = p;
          if (s == 0 && srow) srow[o] = key_score(kx);
        }
        gs[s] += is_gt ? 1u : 0u;
        es[s] += is_eq ? 1u : 0u;
      }
    });
}

struct StreamLayout {
  size_t rows, hist, samp, cnt, above, base, list, cand, total;
};

// nbk: candidate blocks per row (the streaming scan's index_scan_blocks(T),
// the most of any producer)
static StreamLayout stream_layout(int32_t R, int64_t T, int64_t nbk) {
  StreamLayout L;
  size_t off = 0;
  L.rows = off; off += align_up((size_t)R * sizeof(StreamRow), 256);
  L.hist = off; off += align_up((size_t)R * kStreamHistWords * 4, 256);
  L.samp = off; off += align_up((size_t)R * index_sample_words() * 4, 256);
  L.cnt = off; off += align_up((size_t)R * nbk * 4, 256);
  L.above = off; off += align_up((size_t)R * kStreamGroups * 2 * 4, 256);
  L.base = off; off += align_up((size_t)R * kStreamGroups * sizeof(StreamBase), 256);
  L.list = off; off += align_up((size_t)2 * R * kListCap * 8, 256);
  L.cand = off; off += align_up((size_t)R * T * 8 + 64, 256);
  L.total = off;
  return L;
}

static int n_segments(int64_t N) { return (int)((N + kSeg - 1) / kSeg); }

enum Path { kSmall, kCompact, kMultipass };
constexpr int kMaxSeg = 2048;                           // segments per row in the compact path
// candidate-list bytes allowed in the workspace: the lists are sized for the
// worst case (every slot a candidate), R N 16 bytes; up to 16 GB (R N <= 2^30,
// e.g. 4,096 prefill rows x 262,144 positions: 17.3 GB in all, a sixteenth of
// the part's HBM) the compact path runs, 2.2x faster there than the multipass
// path that reads the scores four times (2.55 vs 5.55 ms)
constexpr int64_t kCandBudget = int64_t(1) << 34;
constexpr int64_t kCandBytesPerSlot = 16;             // per-segment and flat (key, position) lists

static int compact_seg(int64_t N) {
  int64_t seg = kSeg;
  while ((N + seg - 1) / seg > kMaxSeg) seg *= 2;
  return (int)seg;
}

static Path choose_path(int32_t R, int64_t N) {
  if (N <= kSmallMax) return kSmall;
  if ((int64_t)R * N * kCandBytesPerSlot <= kCandBudget) return kCompact;
  return kMultipass;
}

struct CompactLayout {
  size_t hist0, seg_cnt, cand_total, state, chunk_cnt, seg_key, seg_pos, cand_key, cand_pos, total;
};

static CompactLayout compact_layout(int32_t R, int64_t N) {
  CompactLayout L;
  const int seg = compact_seg(N);
  const int n_seg = (int)((N + seg - 1) / seg);
  const size_t slots = (size_t)R * N * 4;
  size_t off = 0;
  L.hist0 = off; off += align_up((size_t)R * kTopBins * 4, 256);
  L.seg_cnt = off; off += align_up((size_t)R * n_seg * 4, 256);
  L.cand_total = off; off += align_up((size_t)R * 4, 256);
  L.state = off; off += align_up((size_t)R * sizeof(SelState), 256);
  L.chunk_cnt = off; off += align_up((size_t)R * ((N + kChunk - 1) / kChunk) * 4 * sizeof(uint32_t), 256);
  L.seg_key = off; off += align_up(slots, 256);
  L.seg_pos = off; off += align_up(slots, 256);
  L.cand_key = off; off += align_up(slots, 256);
  L.cand_pos = off; off += align_up(slots, 256);
  L.total = off;
  return L;
}

static size_t ws_layout(int32_t R, int64_t N, size_t* off_state, size_t* off_seg) {
  size_t hist = align_up((size_t)R * kBins * sizeof(uint32_t), 256);
  size_t state = align_up((size_t)R * sizeof(RowState), 256);
  size_t seg = align_up((size_t)R * n_segments(N) * 2 * sizeof(uint32_t), 256);
  if (off_state) *off_state = hist;
  if (off_seg) *off_seg = hist + state;
  return hist + state + seg;
}

static size_t workspace_for(int32_t R, int64_t N) {
  switch (choose_path(R, N)) {
    case kSmall: return 256;
    case kCompact: return compact_layout(R, N).total;
    default: return ws_layout(R, N, nullptr, nullptr);
  }
}

// small path; a second selection (k2 <= k, positions only) when idx2_out is set
static void launch_small(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k,
                         const int32_t* index_map, int32_t* idx_out, float* score_out, hipStream_t s,
                         int32_t k2 = 0, int32_t* idx2_out = nullptr) {
  const int J = (int)((N + kSmallThreads * 4 - 1) / (kSmallThreads * 4));
  if (J <= 1)
    topk_small_kernel<1><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out,
                                                     k2, idx2_out);
  else if (J <= 2)
    topk_small_kernel<2><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out,
                                                     k2, idx2_out);
  else if (J <= 4)
    topk_small_kernel<4><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out,
                                                     k2, idx2_out);
  else
    topk_small_kernel<8><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out,
                                                     k2, idx2_out);
}

// compact path; a second selection (k2 <= k, positions only) when idx2_out is set
static void launch_compact(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k,
                           const int32_t* index_map, int32_t* idx_out, float* score_out, int32_t k2,
                           int32_t* idx2_out, uint8_t* ws, hipStream_t s) {
  const CompactLayout L = compact_layout(R, N);
  const int seg = compact_seg(N);
  const int nseg = (int)((N + seg - 1) / seg);
  uint32_t* hist0 = reinterpret_cast<uint32_t*>(ws + L.hist0);
  uint32_t* seg_cnt = reinterpret_cast<uint32_t*>(ws + L.seg_cnt);
  uint32_t* cand_total = reinterpret_cast<uint32_t*>(ws + L.cand_total);
  uint32_t* seg_key = reinterpret_cast<uint32_t*>(ws + L.seg_key);
  int32_t* seg_pos = reinterpret_cast<int32_t*>(ws + L.seg_pos);
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(ws + L.cand_key);
  int32_t* cand_pos = reinterpret_cast<int32_t*>(ws + L.cand_pos);
  {
    const int64_t nh = (int64_t)R * kTopBins;
    topk_zero_kernel<<<(int)((nh + kThreads - 1) / kThreads), kThreads, 0, s>>>(hist0, nh);
    topk_top_hist_kernel<<<dim3(n_segments(N), R), kThreads, 0, s>>>(scores, N, row_stride, index_map, hist0);
  }
  topk_compact_kernel<<<dim3(nseg, R), kThreads, 0, s>>>(scores, N, row_stride, index_map, k, seg, hist0, seg_key,
                                                         seg_pos, seg_cnt, nseg);
  topk_flatten_kernel<<<dim3(nseg, R), kThreads, 0, s>>>(N, seg, seg_key, seg_pos, seg_cnt, nseg, cand_key, cand_pos,
                                                         cand_total);
  SelState* st = reinterpret_cast<SelState*>(ws + L.state);
  uint32_t* chunk_cnt = reinterpret_cast<uint32_t*>(ws + L.chunk_cnt);
  if (idx2_out) {
    topk_select_cand_kernel<2><<<R, kFinishThreads, 0, s>>>(N, hist0, cand_key, cand_total, k, k2, st, chunk_cnt);
    topk_write_cand_kernel<2><<<dim3(kWriteBlocks, R), kThreads, 0, s>>>(N, cand_key, cand_pos, cand_total, st,
                                                                         chunk_cnt, k, idx_out, score_out, k2,
                                                                         idx2_out);
  } else {
    topk_select_cand_kernel<1><<<R, kFinishThreads, 0, s>>>(N, hist0, cand_key, cand_total, k, 0, st, chunk_cnt);
    topk_write_cand_kernel<1><<<dim3(kWriteBlocks, R), kThreads, 0, s>>>(N, cand_key, cand_pos, cand_total, st,
                                                                         chunk_cnt, k, idx_out, score_out, 0,
                                                                         nullptr);
  }
}

static void launch_multipass(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k,
                             const int32_t* index_map, int32_t* idx_out, float* score_out, uint8_t* ws,
                             hipStream_t s) {
  size_t off_state, off_seg;
  ws_layout(R, N, &off_state, &off_seg);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws);
  RowState* st = reinterpret_cast<RowState*>(ws + off_state);
  uint32_t* seg = reinterpret_cast<uint32_t*>(ws + off_seg);
  const int nseg = n_segments(N);
  dim3 g2(nseg, R);
  topk_init_kernel<<<R, kThreads, 0, s>>>(hist, st);
  topk_hist_kernel<0><<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, hist, st);
  topk_select_kernel<0><<<R, kThreads, 0, s>>>(hist, st, k);
  topk_hist_kernel<1><<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, hist, st);
  topk_select_kernel<1><<<R, kThreads, 0, s>>>(hist, st, k);
  topk_hist_kernel<2><<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, hist, st);
  topk_select_kernel<2><<<R, kThreads, 0, s>>>(hist, st, k);
  topk_count_kernel<<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, st, seg, nseg);
  topk_write_kernel<<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, st, seg, nseg, k, idx_out, score_out);
}

static csa2_status check_scores(const float* scores, int32_t R, int64_t N, int64_t row_stride,
                                const int32_t* index_map) {
  if (!scores) return CSA2_EINVAL;
  if (R <= 0 || N <= 0) return CSA2_EINVAL;
  if (N % 4 != 0 || N >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (row_stride < N || row_stride % 4 != 0) return CSA2_EINVAL;
  if (!aligned(scores, 16) || (index_map && !aligned(index_map, 16))) return CSA2_EALIGN;
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_topk_workspace_size(int32_t R, int64_t N, int32_t k) {
  (void)k;
  if (R <= 0 || N <= 0) return 0;
  return workspace_for(R, N);
}

extern "C" csa2_status csa2_topk(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k,
                                 const int32_t* index_map, int32_t* idx_out, float* score_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  csa2_status st = check_scores(scores, R, N, row_stride, index_map);
  if (st != CSA2_OK) return st;
  if (!idx_out || k <= 0) return CSA2_EINVAL;
  if (!aligned(idx_out, 4) || (score_out && !aligned(score_out, 4))) return CSA2_EALIGN;
  if (!workspace || workspace_bytes < workspace_for(R, N)) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  switch (choose_path(R, N)) {
    case kSmall: launch_small(scores, R, N, row_stride, k, index_map, idx_out, score_out, s); break;
    case kCompact: launch_compact(scores, R, N, row_stride, k, index_map, idx_out, score_out, 0, nullptr, ws, s); break;
    default: launch_multipass(scores, R, N, row_stride, k, index_map, idx_out, score_out, ws, s); break;
  }
  return launch_status();
}

extern "C" size_t csa2_topk_pool_workspace_size(int32_t R, int64_t N, int32_t k_pool) {
  return csa2_topk_workspace_size(R, N, k_pool);
}

extern "C" csa2_status csa2_topk_pool(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k_pool,
                                      int32_t k_top, const int32_t* index_map, int32_t* pool_idx,
                                      float* pool_scores, int32_t* top_idx, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  csa2_status st = check_scores(scores, R, N, row_stride, index_map);
  if (st != CSA2_OK) return st;
  if (!pool_idx || !top_idx || k_pool <= 0 || k_top <= 0 || k_top > k_pool) return CSA2_EINVAL;
  if (!aligned(pool_idx, 4) || !aligned(top_idx, 4) || (pool_scores && !aligned(pool_scores, 4))) return CSA2_EALIGN;
  if (!workspace || workspace_bytes < workspace_for(R, N)) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  switch (choose_path(R, N)) {
    case kSmall:
      launch_small(scores, R, N, row_stride, k_pool, index_map, pool_idx, pool_scores, s, k_top, top_idx);
      break;
    case kCompact:
      launch_compact(scores, R, N, row_stride, k_pool, index_map, pool_idx, pool_scores, k_top, top_idx, ws, s);
      break;
    default:
      launch_multipass(scores, R, N, row_stride, k_pool, index_map, pool_idx, pool_scores, ws, s);
      launch_multipass(scores, R, N, row_stride, k_top, index_map, top_idx, nullptr, ws, s);
      break;
  }
  return launch_status();
}

// Whether csa2_index_full_pool takes its streaming path: rows longer than the
// one-workgroup selection's limit.  Short rows are scored first (into the
// caller's array or the workspace) and csa2_topk_pool selects.
static bool pool_may_stream(int32_t R, int64_t T) { return R > 0 && T > kSmallMax; }

// The streaming selection runs over batches of rows whose candidate storage
// (sized for the worst case, every visible position a candidate: 8 bytes per
// position) fits the workspace.  The size query asks for batches that fit
// kPoolBatchBytes, below 1 GB for any R (4,096 rows x 2^20 positions: 96-row
// batches, 43 of them); a larger workspace runs fewer, larger batches (every
// batch costs about seven launches' fixed time: at 4,096 x 262,144, ten
// batches of 416 rows took 1.79 ms against 1.05 ms for one).  Batches of 32 or
// more rows are whole multiples of 32 (the query-block scan's row block).
constexpr size_t kPoolBatchBytes = size_t(896) << 20;

static size_t stream_bytes(int32_t R, int64_t T) {
  const size_t a = stream_layout(R, T, index_scan_blocks(T)).total;
  const size_t b = stream_layout(R, T, (T + kQueryBlockPositions - 1) / kQueryBlockPositions).total;
  return a > b ? a : b;
}

// the most rows per batch (up to R) whose storage fits `bytes`, at least one
static int32_t stream_batch_rows(int32_t R, int64_t T, size_t bytes) {
  // all rows at once when they fit (the per-row estimate below carries each
  // batch's fixed part once per row, so it alone would split such a workspace)
  if (stream_bytes(R, T) <= bytes) return R;
  int64_t rb = (int64_t)(bytes / stream_bytes(1, T));
  if (rb >= R) rb = R;
  if (rb > 32 && rb < R) rb -= rb % 32;
  while (rb > 1 && stream_bytes((int32_t)rb, T) > bytes) rb -= rb > 32 ? 32 : 1;
  return (int32_t)(rb < 1 ? 1 : rb);
}

extern "C" size_t csa2_index_full_pool_workspace_size(int32_t R, int64_t T, int32_t k_pool) {
  if (R <= 0 || T <= 0) return 0;
  if (pool_may_stream(R, T)) return stream_bytes(stream_batch_rows(R, T, kPoolBatchBytes), T);
  return align_up(csa2_topk_workspace_size(R, T, k_pool), 256) + align_up((size_t)R * T * 4, 256);
}

extern "C" size_t csa2_index_full_pool_batch_workspace_size(int32_t rows_per_batch, int64_t T, int32_t k_pool) {
  if (rows_per_batch <= 0 || T <= 0) return 0;
  if (pool_may_stream(rows_per_batch, T)) return stream_bytes(rows_per_batch, T);
  return csa2_index_full_pool_workspace_size(rows_per_batch, T, k_pool);
}

extern "C" int32_t csa2_index_full_pool_streams(int32_t R, int64_t T) {
  return (R > 0 && T > 0 && pool_may_stream(R, T)) ? 1 : 0;
}

// Streaming selection of R rows (one batch).  Rows of one sequence in runs
// (chunked prefill) share key tiles in the query-block scan, with candidate
// blocks of 1,024 positions; otherwise each row streams its keys, blocks of 128.
// (positions within a block are 32-bit in the query-block scan: rows of up to
// 2^31 - 2^11 positions)
static csa2_status stream_pool_batch(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T,
                              const int32_t* row_seq, const int64_t* row_limit, float* scores, int32_t k_pool,
                              int32_t k_top, int32_t* pool_idx, float* pool_scores, int32_t* top_idx, uint8_t* ws,
                              void* scan_start, void* scan_end, hipStream_t s, const PageMap& pm) {
  const bool qblocks = !index_scan_streams(R, row_seq) && T <= (int64_t(1) << 31) - 2048;
  const int bsz = qblocks ? kQueryBlockPositions : kBlockPositions;
  const int64_t nbk = qblocks ? (T + bsz - 1) / bsz : index_scan_blocks(T);
  const StreamLayout L = stream_layout(R, T, nbk);
  StreamRow* rows = reinterpret_cast<StreamRow*>(ws + L.rows);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
  uint32_t* samp = reinterpret_cast<uint32_t*>(ws + L.samp);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
  uint32_t* above = reinterpret_cast<uint32_t*>(ws + L.above);
  StreamBase* base = reinterpret_cast<StreamBase*>(ws + L.base);
  uint2* list = reinterpret_cast<uint2*>(ws + L.list);
  uint2* cand = reinterpret_cast<uint2*>(ws + L.cand);
  // gather / write workgroups per row: up to 64, fewer when many rows fill the chip anyway
  const int groups = (int)std::min<int64_t>(std::min<int64_t>(kStreamGroups, nbk), std::max<int64_t>(1, 4096 / R));
  const int bpw = (int)((nbk + groups - 1) / groups);
  // the per-row scan derives each row's threshold from the sample itself when each of its workgroups
  // serves one row; otherwise (and for the query-block scan) the threshold kernel does
  const bool scan_tau = !qblocks && index_scan_derives_tau(R);
  launch_index_sample_tau(q_idx, k_idx, R, T, row_seq, row_limit, k_pool, rows, hist, samp, !scan_tau, s, pm);
  if (scan_start && hipEventRecord((hipEvent_t)scan_start, s) != hipSuccess) return CSA2_ELAUNCH;
  const CandOut co{rows, hist, cand, cnt, nbk, scan_tau ? samp : nullptr, k_pool};
  if (qblocks) {
    launch_index_block_cand(q_idx, k_idx, R, T, row_seq, row_limit, scores, co, bsz, s, pm);
    stream_hist_kernel<<<R, kSG, 0, s>>>(T, nbk, bsz, rows, hist, cand, cnt);
  } else {
    launch_index_scan(q_idx, k_idx, R, T, row_seq, row_limit, scores, &co, s, pm);
  }
  if (scan_end && hipEventRecord((hipEvent_t)scan_end, s) != hipSuccess) return CSA2_ELAUNCH;
  stream_gather_kernel<<<dim3(groups, R), kSG, 0, s>>>(q_idx, k_idx, T, row_seq, row_limit, nbk, bpw, bsz, rows,
                                                       hist, cand, cnt, above, list, base, k_pool, k_top, pm);
  stream_write_kernel<<<dim3(groups, R), kSG, 0, s>>>(T, nbk, bpw, bsz, rows, base, cand, cnt, k_pool, k_top,
                                                      pool_idx, pool_scores, top_idx);
  return launch_status();
}

static csa2_status index_full_pool(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B, int64_t T,
                                   const int32_t* row_seq, const int64_t* row_limit, float* scores, int32_t k_pool,
                                   int32_t k_top, int32_t* pool_idx, float* pool_scores, int32_t* top_idx,
                                   void* workspace, size_t workspace_bytes, void* scan_start, void* scan_end,
                                   void* stream, const PageMap& pm) {
  if (!q_idx || !k_idx || !pool_idx || !top_idx) return CSA2_EINVAL;
  if (R <= 0 || B <= 0 || T <= 0 || k_pool <= 0 || k_top <= 0 || k_top > k_pool) return CSA2_EINVAL;
  if (!row_seq && R != B) return CSA2_EINVAL;
  if (T % 4 != 0 || T >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || (scores && !aligned(scores, 16)) || !aligned(pool_idx, 4) ||
      !aligned(top_idx, 4) || (pool_scores && !aligned(pool_scores, 4)))
    return CSA2_EALIGN;
  if (!workspace || workspace_bytes < csa2_index_full_pool_workspace_size(R, T, k_pool)) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  {
    const csa2_status dc = debug_check(row_seq, R, B, nullptr, nullptr, 0, 0, nullptr, 0, T, s);
    if (dc != CSA2_OK) return dc;
  }
  if (!pool_may_stream(R, T)) {
    // short rows or very long R x T: scores first (into the workspace when the
    // caller takes none), then the selection
    const size_t tk = align_up(csa2_topk_workspace_size(R, T, k_pool), 256);
    float* sc = scores ? scores : reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + tk);
    if (scan_start && hipEventRecord((hipEvent_t)scan_start, s) != hipSuccess) return CSA2_ELAUNCH;
    csa2_status st = CSA2_OK;
    if (pm.table) {
      launch_index_scan(q_idx, k_idx, R, T, row_seq, row_limit, sc, nullptr, s, pm);
      st = launch_status();
    } else {
      st = csa2_index_full(q_idx, k_idx, R, B, T, row_seq, row_limit, sc, stream);
    }
    if (st != CSA2_OK) return st;
    if (scan_end && hipEventRecord((hipEvent_t)scan_end, s) != hipSuccess) return CSA2_ELAUNCH;
    return csa2_topk_pool(sc, R, T, T, k_pool, k_top, nullptr, pool_idx, pool_scores, top_idx, workspace, tk,
                          stream);
  }
  // Streaming selection in batches of rows.  A batch without row_seq starts at
  // sequence r0: its keys (dense) or its block-table rows (paged) are offset.
  // The scan events bracket the first batch's scan start and the last one's end.
  const int32_t rb = stream_batch_rows(R, T, workspace_bytes);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int32_t r0 = 0; r0 < R; r0 += rb) {
    const int32_t n = std::min(rb, R - r0);
    const uint8_t* kb = k_idx;
    PageMap pb = pm;
    if (!row_seq) {
      if (pm.table) pb.table = pm.table + (int64_t)r0 * pm.max_blocks;
      else kb = k_idx + (int64_t)r0 * T * kIndexDim;
    }
    const csa2_status st = stream_pool_batch(
        q_idx + (int64_t)r0 * kIndexDim, kb, n, T, row_seq ? row_seq + r0 : nullptr,
        row_limit ? row_limit + r0 : nullptr, scores ? scores + (int64_t)r0 * T : nullptr, k_pool, k_top,
        pool_idx + (int64_t)r0 * k_pool, pool_scores ? pool_scores + (int64_t)r0 * k_pool : nullptr,
        top_idx + (int64_t)r0 * k_top, ws, r0 == 0 ? scan_start : nullptr, r0 + n >= R ? scan_end : nullptr, s, pb);
    if (st != CSA2_OK) return st;
  }
  return CSA2_OK;
}

extern "C" csa2_status csa2_index_full_pool(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B,
                                            int64_t T, const int32_t* row_seq, const int64_t* row_limit,
                                            float* scores, int32_t k_pool, int32_t k_top, int32_t* pool_idx,
                                            float* pool_scores, int32_t* top_idx, void* workspace,
                                            size_t workspace_bytes, void* scan_start, void* scan_end,
                                            void* stream) {
  return index_full_pool(q_idx, k_idx, R, B, T, row_seq, row_limit, scores, k_pool, k_top, pool_idx, pool_scores,
                         top_idx, workspace, workspace_bytes, scan_start, scan_end, stream, PageMap{});
}

extern "C" size_t csa2_index_full_pool_paged_workspace_size(int32_t R, int64_t T, int32_t k_pool) {
  return csa2_index_full_pool_workspace_size(R, T, k_pool);
}

extern "C" csa2_status csa2_index_full_pool_paged(const uint8_t* q_idx, const uint8_t* k_pages, int32_t R, int32_t B,
                                                  int64_t T, const int32_t* row_seq, const int64_t* row_limit,
                                                  const int32_t* block_table, int64_t max_blocks, int32_t page,
                                                  float* scores, int32_t k_pool, int32_t k_top, int32_t* pool_idx,
                                                  float* pool_scores, int32_t* top_idx, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  csa2_status st = check_pages(block_table, max_blocks, page, T);
  if (st != CSA2_OK) return st;
  return index_full_pool(q_idx, k_pages, R, B, T, row_seq, row_limit, scores, k_pool, k_top, pool_idx, pool_scores,
                         top_idx, workspace, workspace_bytes, nullptr, nullptr, stream,
                         PageMap{block_table, max_blocks, page});
}
