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
#include "common.hpp"

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

__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = x == 0.0f ? 0u : __float_as_uint(x);     // -0 ranks equal to +0
  if (x != x || x == -__builtin_inff()) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// inverse of score_key for visible keys (a -0 score comes back as +0)
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

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

// block-wide exclusive prefix sum of one value per thread (256 threads)
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp /* >= 4 */, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return base + x - v;
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

// block-wide exclusive prefix sum, 1024 threads (16 waves); wt holds >= 16 words
__device__ __forceinline__ uint32_t block_scan_1024(uint32_t v, uint32_t* wt, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) wt[wave] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t t = wt[w];
    base += w < wave ? t : 0u;
    tot += t;
  }
  total = tot;
  __syncthreads();
  return base + inc - v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Wave w owns the slots [256 J w, 256 J (w+1)) of the row, 4096 J >= N;
// in step it, lane l holds slots 256 (J w + it) + 4l + [0, 4).  So every wave
// reads 1 KiB runs, and the ordered write walks the row in slot order with
// ballot prefix counts.  The radix digits are 12 bits wide and start at the
// highest bit in which the row's visible keys differ.
template <int J>
__global__ void __launch_bounds__(kSmallThreads)
topk_small_kernel(const float* __restrict__ scores, int N, int64_t stride, const int32_t* __restrict__ index_map,
                  int32_t k, int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  __shared__ uint32_t h[kSmallBins];
  __shared__ uint32_t wt[16], wt2[16];
  __shared__ uint32_t red[3][16];
  __shared__ uint32_t s_digit, s_above;
  __shared__ __attribute__((aligned(16))) int32_t s_map[J * kSmallThreads * 4];   // index_map row (if any)
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wbase = wave * J * 256;
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;

  uint32_t key[J][4];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nvis = 0u;
  {
    float4 v[J];
    int4 mp[J];
#pragma unroll
    for (int it = 0; it < J; ++it) {
      const int s = wbase + it * 256 + 4 * lane;
      const bool in = s < N;
      v[it] = in ? *reinterpret_cast<const float4*>(row + s) : make_float4(0.f, 0.f, 0.f, 0.f);
      mp[it] = in ? (map_row ? *reinterpret_cast<const int4*>(map_row + s) : make_int4(0, 0, 0, 0))
                  : make_int4(-1, -1, -1, -1);
    }
#pragma unroll
    for (int it = 0; it < J; ++it) {
      const float f[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
      const int32_t m4[4] = {mp[it].x, mp[it].y, mp[it].z, mp[it].w};
      if (map_row) *reinterpret_cast<int4*>(s_map + wbase + it * 256 + 4 * lane) = mp[it];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kk = m4[j] < 0 ? 0u : score_key(f[j]);
        key[it][j] = kk;
        if (kk != 0u) {
          kmin = min(kmin, kk);
          kmax = max(kmax, kk);
          ++nvis;
        }
      }
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  nvis = wave_sum_u32(nvis);
  if (lane == 0) { red[0][wave] = kmin; red[1][wave] = kmax; red[2][wave] = nvis; }
  __syncthreads();
  kmin = 0xFFFFFFFFu; kmax = 0u; nvis = 0u;
#pragma unroll
  for (int w = 0; w < 16; ++w) { kmin = min(kmin, red[0][w]); kmax = max(kmax, red[1][w]); nvis += red[2][w]; }
  kmin = uniform_u32(kmin);
  kmax = uniform_u32(kmax);
  nvis = uniform_u32(nvis);
  const uint32_t k_eff = nvis < (uint32_t)k ? nvis : (uint32_t)k;

  // radix select of tau, the k_eff-th largest visible key
  uint32_t need = k_eff, prefix = 0u;
  if (k_eff > 0) {
    // bits shared by every visible key: those above the highest set bit of
    // kmin ^ kmax.  Smearing the difference down avoids a select on
    // kmin == kmax: this compiler's post-RA instruction shrinking can drop the
    // exec-mask AND whose SCC such a select reads.
    uint32_t below = kmin ^ kmax;
    below |= below >> 1;
    below |= below >> 2;
    below |= below >> 4;
    below |= below >> 8;
    below |= below >> 16;
    prefix = kmax & ~below;
    int hi = __popc(below) - 1;             // highest unresolved bit (below = 2^(hi+1) - 1), -1 if none
#pragma unroll 1
    while (hi >= 0) {
      const int width = hi + 1 < kSmallBits ? hi + 1 : kSmallBits;
      const int shift = hi + 1 - width;
      const uint32_t bmask = (1u << width) - 1u;
      const uint32_t hp = hi >= 31 ? 0u : (prefix >> (hi + 1));
      for (int i = tid; i < kSmallBins; i += kSmallThreads) h[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int it = 0; it < J; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t kk = key[it][j];
          const bool match = kk != 0u && (hi >= 31 || (kk >> (hi + 1)) == hp);
          if (match) atomicAdd(&h[(kk >> shift) & bmask], 1u);
        }
      }
      __syncthreads();
      // thread t owns bins kSmallBins-1-4t-j (j = 0..3): a descending walk
      uint32_t c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = h[kSmallBins - 1 - 4 * tid - j];
        local += c[j];
      }
      uint32_t total;
      const uint32_t excl = block_scan_1024(local, wt, total);
      if (excl < need && need <= excl + local) {
        uint32_t acc = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (acc < need && need <= acc + c[j]) {
            s_digit = (uint32_t)(kSmallBins - 1 - 4 * tid - j);
            s_above = acc;
          }
          acc += c[j];
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      need -= s_above;
      hi = shift - 1;
    }
  }
  const uint32_t tau = prefix, need_eq = need;

  // ordered write: a slot's output index is (#keys > tau before it) + min(#keys == tau before it, need_eq)
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int it = 0; it < J; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t kk = key[it][j];
      n_gt += kk != 0u && kk > tau;
      n_eq += kk != 0u && kk == tau;
    }
  n_gt = wave_sum_u32(n_gt);
  n_eq = wave_sum_u32(n_eq);
  if (lane == 0) { wt[wave] = n_gt; wt2[wave] = n_eq; }
  __syncthreads();
  uint32_t G = 0, E = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    G += w < wave ? wt[w] : 0u;
    E += w < wave ? wt2[w] : 0u;
  }
  int32_t* orow = idx_out + (int64_t)r * k;
  float* srow = score_out ? score_out + (int64_t)r * k : nullptr;
  if (k_eff > 0) {
#pragma unroll
    for (int it = 0; it < J; ++it) {
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kk = key[it][j];
        cg += kk != 0u && kk > tau;
        ce += kk != 0u && kk == tau;
      }
      uint32_t tg, te;
      const int s = wbase + it * 256 + 4 * lane;
      uint32_t g = G + wave_exclusive_small(cg, tg);
      uint32_t e = E + wave_exclusive_small(ce, te);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kk = key[it][j];
        const bool is_gt = kk != 0u && kk > tau;
        const bool is_eq = kk != 0u && kk == tau;
        const bool take = is_gt || (is_eq && e < need_eq);
        const uint32_t o = g + (is_gt ? min(e, need_eq) : e);
        const int32_t pv = map_row ? s_map[s + j] : s + j;
        g += is_gt ? 1u : 0u;
        e += is_eq ? 1u : 0u;
        if (take && o < k_eff) {
          orow[o] = pv;
          if (srow) srow[o] = key_score(kk);
        }
      }
      G += tg;
      E += te;
    }
  }
  for (int i = (int)k_eff + tid; i < k; i += kSmallThreads) {
    orow[i] = -1;
    if (srow) srow[i] = __builtin_nanf("");
  }
}

// ----------------------------------------------------------------------------
// compact path
// ----------------------------------------------------------------------------
struct CompactState {
  uint32_t b0;          // top digit of tau
  uint32_t k_eff;
  uint32_t tau;
  uint32_t need_eq;
  int32_t tie_slot_max; // equal keys at slots <= this are selected
  uint32_t pad[3];
};

__global__ void __launch_bounds__(kThreads)
topk_cinit_kernel(uint32_t* __restrict__ hist0, uint32_t* __restrict__ cand_count) {
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist0[(int64_t)r * kBins + i] = 0u;
  if (threadIdx.x == 0) cand_count[r] = 0u;
}

// derive (b0, need within bin b0, k_eff) from the row's top-digit histogram, 256 threads
__device__ __forceinline__ void derive_b0(const uint32_t* g, int32_t k, uint32_t* tmp, uint32_t& b0, uint32_t& need1,
                                          uint32_t& k_eff) {
  __shared__ uint32_t s_digit, s_above;
  uint32_t c[8];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int bin = kBins - 1 - (threadIdx.x * 8 + j);
    c[j] = bin == 0 ? 0u : g[bin];
    local += c[j];
  }
  uint32_t total;
  uint32_t excl = block_exclusive_scan(local, tmp, total);
  uint32_t need = total < (uint32_t)k ? total : (uint32_t)k;
  if (threadIdx.x == 0) { s_digit = 0xFFFFFFFFu; s_above = 0u; }
  __syncthreads();
  if (need > 0 && excl < need && need <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (acc < need && need <= acc + c[j]) { s_digit = (uint32_t)(kBins - 1 - (threadIdx.x * 8 + j)); s_above = acc; }
      acc += c[j];
    }
  }
  __syncthreads();
  k_eff = need;
  b0 = s_digit;
  need1 = need - s_above;
  __syncthreads();
}

// per segment: count keys above bin b0, append keys inside bin b0 to the candidates
// (one atomic per 8192-slot block: thread t scans 32 consecutive slots)
constexpr int kCompactBlock = kThreads * 32;

__global__ void __launch_bounds__(kThreads)
topk_compact_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                    int32_t k, int seg, const uint32_t* __restrict__ hist0, uint32_t* __restrict__ cand_count,
                    uint2* __restrict__ cand, int64_t cand_cap, uint32_t* __restrict__ seg_gt, int n_seg) {
  __shared__ uint32_t tmp[8];
  __shared__ uint32_t s_base;
  const int r = blockIdx.y;
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int64_t s0 = (int64_t)blockIdx.x * seg;
  const int64_t s1 = min(N, s0 + seg);
  uint2* crow = cand + (int64_t)r * cand_cap;
  // thread t scans 32 consecutive slots per block; the first block's loads are
  // issued before the threshold bin is derived from the histogram
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
      keys[4 * q + 0] = (!in || mp[q].x < 0) ? 0u : score_key(v[q].x);
      keys[4 * q + 1] = (!in || mp[q].y < 0) ? 0u : score_key(v[q].y);
      keys[4 * q + 2] = (!in || mp[q].z < 0) ? 0u : score_key(v[q].z);
      keys[4 * q + 3] = (!in || mp[q].w < 0) ? 0u : score_key(v[q].w);
    }
  };
  uint32_t keys[32];
  load32(s0 + (int64_t)threadIdx.x * 32, keys);
  uint32_t b0, need1, k_eff;
  derive_b0(hist0 + (int64_t)r * kBins, k, tmp, b0, need1, k_eff);
  uint32_t gt = 0;
  if (k_eff > 0) {
    for (int64_t blk = s0; blk < s1; blk += kCompactBlock) {
      const int64_t i0 = blk + (int64_t)threadIdx.x * 32;
      if (blk != s0) load32(i0, keys);
      uint32_t nc = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t d0 = keys[j] >> 21;
        gt += keys[j] != 0u && d0 > b0;
        nc += keys[j] != 0u && d0 == b0;
      }
      uint32_t total;
      uint32_t off = block_exclusive_scan(nc, tmp, total);
      if (threadIdx.x == 0) s_base = total ? atomicAdd(&cand_count[r], total) : 0u;
      __syncthreads();
      uint32_t p = s_base + off;
      if (nc) {
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (keys[j] != 0u && (keys[j] >> 21) == b0) crow[p++] = make_uint2((uint32_t)(i0 + j), keys[j]);
      }
      __syncthreads();
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) gt += __shfl_xor(gt, o, 64);
  if (lane == 0) tmp[wave] = gt;
  __syncthreads();
  if (threadIdx.x == 0) seg_gt[(int64_t)r * n_seg + blockIdx.x] = tmp[0] + tmp[1] + tmp[2] + tmp[3];
}

// one workgroup per row: finish the selection on the candidates
constexpr int kMaxSeg = 2048;

__global__ void __launch_bounds__(1024)
topk_refine_kernel(int32_t k, int seg, const uint32_t* __restrict__ hist0, const uint32_t* __restrict__ cand_count,
                   const uint2* __restrict__ cand, int64_t cand_cap, const uint32_t* __restrict__ seg_gt,
                   uint32_t* __restrict__ seg_off, int n_seg, CompactState* __restrict__ st) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t tmp[32];
  __shared__ uint32_t s_digit, s_above;
  __shared__ uint32_t sc[kMaxSeg];
  __shared__ uint32_t s_b0, s_need1, s_keff;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  // b0 / need1 / k_eff from the top-digit histogram (1024-thread version)
  for (int i = tid; i < kBins; i += 1024) h[i] = hist0[(int64_t)r * kBins + i];
  __syncthreads();
  uint32_t total;
  find_digit_1024(h, 0xFFFFFFFFu, true, tmp, &s_digit, &s_above, total);
  {
    uint32_t k_eff = total < (uint32_t)k ? total : (uint32_t)k;
    find_digit_1024(h, k_eff, true, tmp, &s_digit, &s_above, total);
    if (tid == 0) { s_keff = k_eff; s_b0 = s_digit; s_need1 = k_eff - s_above; }
    __syncthreads();
  }
  const uint32_t k_eff = s_keff, b0 = s_b0;
  uint32_t need = s_need1;
  const uint32_t nc = cand_count[r];
  const uint2* crow = cand + (int64_t)r * cand_cap;
  uint32_t prefix = b0 << 21;
  bool none = (k_eff == 0) || (b0 == 0xFFFFFFFFu);
  if (none) prefix = 0xFFFFFFFFu;
#pragma unroll 1
  for (int d = 1; d < 3 && !none; ++d) {
    for (int i = tid; i < kBins; i += 1024) h[i] = 0u;
    __syncthreads();
    const uint32_t mask = digit_mask_above(d);
    const int shift = digit_shift(d);
    for (uint32_t b = 0; b < nc; b += 8 * 1024) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = b + u * 1024 + tid;
        kk[u] = i < nc ? crow[i].y : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b + u * 1024 + tid < nc && (kk[u] & mask) == prefix) atomicAdd(&h[(kk[u] >> shift) & (kBins - 1)], 1u);
    }
    __syncthreads();
    find_digit_1024(h, need, false, tmp, &s_digit, &s_above, total);
    if (s_digit == 0xFFFFFFFFu) { none = true; prefix = 0xFFFFFFFFu; need = 0; break; }
    prefix |= s_digit << shift;
    need -= s_above;
  }
  const uint32_t tau = prefix, need_eq = none ? 0u : need;
  // ties: the need_eq lowest slots among candidates with key == tau -> largest selected slot
  int32_t tie_max = -1;
  if (!none) {
    uint32_t n_tie = 0;
    for (uint32_t b = 0; b < nc; b += 8 * 1024) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = b + u * 1024 + tid;
        kk[u] = i < nc ? crow[i].y : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) n_tie += (b + u * 1024 + tid < nc) && kk[u] == tau;
    }
    uint32_t tot;
    block_exclusive_scan_1024(n_tie, tmp, tot);
    if (tot <= need_eq) {
      tie_max = 0x7FFFFFFF;
    } else {
      // radix select of the need_eq-th smallest slot among the ties (slots < 2^31; digits of 11/10/10 bits)
      uint32_t sprefix = 0, sneed = need_eq;
      const int shifts[3] = {20, 10, 0};
      const uint32_t masks[3] = {0u, 0xFFF00000u, 0xFFFFFC00u};
#pragma unroll 1
      for (int d = 0; d < 3; ++d) {
        for (int i = tid; i < kBins; i += 1024) h[i] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < nc; i += 1024) {
          uint2 c = crow[i];
          if (c.y == tau && (c.x & masks[d]) == sprefix) atomicAdd(&h[(c.x >> shifts[d]) & (kBins - 1)], 1u);
        }
        __syncthreads();
        // ascending search: thread t owns bins 2t, 2t+1
        const uint32_t c0 = h[2 * tid], c1 = h[2 * tid + 1];
        uint32_t t2;
        uint32_t ex = block_exclusive_scan_1024(c0 + c1, tmp, t2);
        if (tid == 0) { s_digit = 0xFFFFFFFFu; s_above = 0u; }
        __syncthreads();
        if (ex < sneed && sneed <= ex + c0) { s_digit = 2 * tid; s_above = ex; }
        else if (ex + c0 < sneed && sneed <= ex + c0 + c1) { s_digit = 2 * tid + 1; s_above = ex + c0; }
        __syncthreads();
        sprefix |= s_digit << shifts[d];
        sneed -= s_above;
        __syncthreads();
      }
      tie_max = (int32_t)sprefix;
    }
  }
  // per-segment selected counts -> output offsets
  for (int i = tid; i < n_seg; i += 1024) sc[i] = seg_gt[(int64_t)r * n_seg + i];
  __syncthreads();
  if (!none)
    for (uint32_t b = 0; b < nc; b += 8 * 1024) {
      uint2 cc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = b + u * 1024 + tid;
        cc[u] = i < nc ? crow[i] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool take = (b + u * 1024 + tid < nc) &&
                          (cc[u].y > tau || (cc[u].y == tau && (int32_t)cc[u].x <= tie_max));
        if (take) atomicAdd(&sc[cc[u].x / seg], 1u);
      }
    }
  __syncthreads();
  // exclusive scan over segments (n_seg <= 2048: two per thread)
  {
    const uint32_t a0 = 2 * tid < n_seg ? sc[2 * tid] : 0u;
    const uint32_t a1 = 2 * tid + 1 < n_seg ? sc[2 * tid + 1] : 0u;
    uint32_t tot;
    uint32_t ex = block_exclusive_scan_1024(a0 + a1, tmp, tot);
    if (2 * tid < n_seg) seg_off[(int64_t)r * n_seg + 2 * tid] = ex;
    if (2 * tid + 1 < n_seg) seg_off[(int64_t)r * n_seg + 2 * tid + 1] = ex + a0;
  }
  if (tid == 0) {
    CompactState cs;
    cs.b0 = none ? 0xFFFFFFFFu : b0;
    cs.k_eff = k_eff;
    cs.tau = tau;
    cs.need_eq = need_eq;
    cs.tie_slot_max = tie_max;
    cs.pad[0] = cs.pad[1] = cs.pad[2] = 0;
    st[r] = cs;
  }
}

// ordered write: thread t owns the 4*E consecutive slots of its part of the segment
__global__ void __launch_bounds__(kThreads)
topk_cwrite_kernel(const float* __restrict__ scores, int64_t N, int64_t stride, const int32_t* __restrict__ index_map,
                   int seg, const CompactState* __restrict__ st, const uint32_t* __restrict__ seg_off, int n_seg,
                   int32_t k, int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  __shared__ uint32_t tmp[8];
  const int r = blockIdx.y;
  const CompactState cs = st[r];
  int32_t* orow = idx_out + (int64_t)r * k;
  float* srow = score_out ? score_out + (int64_t)r * k : nullptr;
  if (blockIdx.x == n_seg - 1) {
    for (int i = (int)cs.k_eff + threadIdx.x; i < k; i += kThreads) {
      orow[i] = -1;
      if (srow) srow[i] = __builtin_nanf("");
    }
  }
  if (cs.k_eff == 0) return;
  const float* row = scores + (int64_t)r * stride;
  const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
  const int64_t s0 = (int64_t)blockIdx.x * seg;
  const int64_t s1 = min(N, s0 + seg);
  auto selected = [&](int64_t i, uint32_t key) -> bool {
    if (key == 0u) return false;
    if ((key >> 21) != cs.b0) return (key >> 21) > cs.b0;
    return key > cs.tau || (key == cs.tau && (int32_t)i <= cs.tie_slot_max);
  };
  uint32_t base = seg_off[(int64_t)r * n_seg + blockIdx.x];
  // blocks of 8192 slots: thread t owns 32 consecutive slots, keys and map values stay in registers
  for (int64_t blk = s0; blk < s1; blk += kCompactBlock) {
    const int64_t i0 = blk + (int64_t)threadIdx.x * 32;
    float4 v[8];
    int4 mp[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t i = i0 + 4 * q;
      v[q] = i < s1 ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      mp[q] = (map_row && i < s1) ? *reinterpret_cast<const int4*>(map_row + i) : make_int4(0, 0, 0, 0);
    }
    uint32_t keys[32];
    int32_t pos[32];
    uint32_t n = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = i0 + 4 * q < s1;
      const float f[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      const int32_t mv[4] = {mp[q].x, mp[q].y, mp[q].z, mp[q].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t i = i0 + 4 * q + j;
        keys[4 * q + j] = (!in || mv[j] < 0) ? 0u : score_key(f[j]);
        pos[4 * q + j] = map_row ? mv[j] : (int32_t)i;
        n += selected(i, keys[4 * q + j]);
      }
    }
    uint32_t tot;
    uint32_t p = base + block_exclusive_scan(n, tmp, tot);
    base += tot;
    if (n) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (selected(i0 + j, keys[j]) && p < cs.k_eff) {
          orow[p] = pos[j];
          if (srow) srow[p] = key_score(keys[j]);
          ++p;
        }
      }
    }
  }
}

static int n_segments(int64_t N) { return (int)((N + kSeg - 1) / kSeg); }

enum Path { kSmall, kCompact, kMultipass };
constexpr int64_t kCandBudget = int64_t(1) << 30;     // candidate-list bytes allowed in the workspace

static int compact_seg(int64_t N) {
  int64_t seg = kSeg;
  while ((N + seg - 1) / seg > kMaxSeg) seg *= 2;
  return (int)seg;
}

static Path choose_path(int32_t R, int64_t N) {
  if (N <= kSmallMax) return kSmall;
  if ((int64_t)R * N * (int64_t)sizeof(uint2) <= kCandBudget) return kCompact;
  return kMultipass;
}

struct CompactLayout {
  size_t hist0, cand_count, seg_gt, seg_off, state, cand, total;
};

static CompactLayout compact_layout(int32_t R, int64_t N) {
  CompactLayout L;
  const int n_seg = (int)((N + compact_seg(N) - 1) / compact_seg(N));
  size_t off = 0;
  L.hist0 = off; off += align_up((size_t)R * kBins * 4, 256);
  L.cand_count = off; off += align_up((size_t)R * 4, 256);
  L.seg_gt = off; off += align_up((size_t)R * n_seg * 4, 256);
  L.seg_off = off; off += align_up((size_t)R * n_seg * 4, 256);
  L.state = off; off += align_up((size_t)R * sizeof(CompactState), 256);
  L.cand = off; off += align_up((size_t)R * N * sizeof(uint2), 256);
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
  if (!scores || !idx_out) return CSA2_EINVAL;
  if (R <= 0 || N <= 0 || k <= 0) return CSA2_EINVAL;
  if (N % 4 != 0 || N >= (int64_t(1) << 31)) return CSA2_ESHAPE;
  if (row_stride < N || row_stride % 4 != 0) return CSA2_EINVAL;
  if (!aligned(scores, 16) || (index_map && !aligned(index_map, 16)) || !aligned(idx_out, 4))
    return CSA2_EALIGN;
  const size_t need = workspace_for(R, N);
  if (!workspace || workspace_bytes < need) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const Path path = choose_path(R, N);
  if (path == kSmall) {
    const int J = (int)((N + kSmallThreads * 4 - 1) / (kSmallThreads * 4));
    if (J <= 1)
      topk_small_kernel<1><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out);
    else if (J <= 2)
      topk_small_kernel<2><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out);
    else if (J <= 4)
      topk_small_kernel<4><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out);
    else
      topk_small_kernel<8><<<R, kSmallThreads, 0, s>>>(scores, (int)N, row_stride, index_map, k, idx_out, score_out);
    return launch_status();
  }
  if (path == kCompact) {
    const CompactLayout L = compact_layout(R, N);
    const int seg = compact_seg(N);
    const int nseg = (int)((N + seg - 1) / seg);
    uint32_t* hist0 = reinterpret_cast<uint32_t*>(ws + L.hist0);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + L.cand_count);
    uint32_t* seg_gt = reinterpret_cast<uint32_t*>(ws + L.seg_gt);
    uint32_t* seg_off = reinterpret_cast<uint32_t*>(ws + L.seg_off);
    CompactState* st = reinterpret_cast<CompactState*>(ws + L.state);
    uint2* cand = reinterpret_cast<uint2*>(ws + L.cand);
    dim3 g2(nseg, R);
    topk_cinit_kernel<<<R, kThreads, 0, s>>>(hist0, cnt);
    topk_hist_kernel<0><<<dim3(n_segments(N), R), kThreads, 0, s>>>(scores, N, row_stride, index_map, hist0, nullptr);
    topk_compact_kernel<<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, k, seg, hist0, cnt, cand, N, seg_gt,
                                                nseg);
    topk_refine_kernel<<<R, 1024, 0, s>>>(k, seg, hist0, cnt, cand, N, seg_gt, seg_off, nseg, st);
    topk_cwrite_kernel<<<g2, kThreads, 0, s>>>(scores, N, row_stride, index_map, seg, st, seg_off, nseg, k, idx_out,
                                               score_out);
    return launch_status();
  }
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
  return launch_status();
}
