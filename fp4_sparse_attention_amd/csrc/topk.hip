// Top-K selection by radix select over order-preserving 32-bit keys.
//
// The HN summary's key points describe CSA2 layers sharing one set of Top-K
// indices and a shallow-layer candidate pool that bounds the deeper layers'
// search; the MarkTechPost retelling (CSA2 paragraph) bounds that pool at
// 16,384 positions.  Selection rule: the k largest visible scores, equal scores
// to the lower slot, output ascending, -1 padding.
//
// Each score maps to a key that orders like the float (sign flip for
// positives, bitwise not for negatives); invisible slots (-inf, NaN, or a
// negative index_map entry) map to key 0, which no visible score reaches
// (the smallest, -FLT_MAX, maps to 0x00800000).  Three digit passes (11, 11 and
// 10 bits) find the k-th largest key tau and how many slots equal to tau are
// still needed; every pass is a segmented histogram (LDS atomics, then one
// global atomic per non-empty bin and workgroup) followed by a one-workgroup
// scan.  A counting pass and an ordered write pass then emit the selected slots
// in slot order, so the output is sorted without a sort and ties go to the
// lowest slots.  All integer work: the result is deterministic.
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
  const RowState s = st[r];
  const bool live = (D == 0) || s.need > 0;
  if (live) {
    const float* row = scores + (int64_t)r * stride;
    const int32_t* map_row = index_map ? index_map + (int64_t)r * N : nullptr;
    const uint32_t mask = digit_mask_above(D);
    const int shift = digit_shift(D);
    const int64_t b0 = (int64_t)blockIdx.x * kSeg;
    const int64_t b1 = min(N, b0 + kSeg);
    for (int64_t i = b0 + threadIdx.x * 4; i < b1; i += kThreads * 4) {
      // N is a multiple of 4, so a 4-slot group never straddles the row end
      float4 v = *reinterpret_cast<const float4*>(row + i);
      int4 mp = map_row ? *reinterpret_cast<const int4*>(map_row + i) : make_int4(0, 0, 0, 0);
      uint32_t k4[4] = {score_key(v.x), score_key(v.y), score_key(v.z), score_key(v.w)};
      int m4[4] = {mp.x, mp.y, mp.z, mp.w};
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

static int n_segments(int64_t N) { return (int)((N + kSeg - 1) / kSeg); }

static size_t ws_layout(int32_t R, int64_t N, size_t* off_state, size_t* off_seg) {
  size_t hist = align_up((size_t)R * kBins * sizeof(uint32_t), 256);
  size_t state = align_up((size_t)R * sizeof(RowState), 256);
  size_t seg = align_up((size_t)R * n_segments(N) * 2 * sizeof(uint32_t), 256);
  if (off_state) *off_state = hist;
  if (off_seg) *off_seg = hist + state;
  return hist + state + seg;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_topk_workspace_size(int32_t R, int64_t N, int32_t k) {
  (void)k;
  if (R <= 0 || N <= 0) return 0;
  return ws_layout(R, N, nullptr, nullptr);
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
  size_t off_state, off_seg;
  size_t need = ws_layout(R, N, &off_state, &off_seg);
  if (!workspace || workspace_bytes < need) return CSA2_EWORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_EALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws);
  RowState* st = reinterpret_cast<RowState*>(ws + off_state);
  uint32_t* seg = reinterpret_cast<uint32_t*>(ws + off_seg);
  hipStream_t s = (hipStream_t)stream;
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
