// Library-wide entry points: ABI version and status strings; the opt-in
// argument validation the entry points share.
#include <stdlib.h>

#include "internal.hpp"

namespace csa2 {

// The validation's result word, one per GPU; its device address is resolved
// once per device (the name is a host-side stand-in, never passed to a kernel).
static __device__ __align__(16) uint32_t dbg_bad;
static std::atomic<uint32_t*> dbg_bad_dev[kMaxDevices];

// One workgroup: every thread checks a strided share of the entries; the
// verdict (1 = a bad entry) is written to *out by thread 0.
__global__ void __launch_bounds__(256)
debug_check_kernel(const int32_t* __restrict__ row_seq, int R, int B, const int32_t* __restrict__ swa_start,
                   const int32_t* __restrict__ swa_len, int64_t n_win, int S, const int32_t* __restrict__ idx,
                   int64_t n_idx, int64_t T, uint32_t* __restrict__ out) {
  __shared__ uint32_t bad;
  if (threadIdx.x == 0) bad = 0u;
  __syncthreads();
  uint32_t mine = 0u;
  if (row_seq)
    for (int i = threadIdx.x; i < R; i += blockDim.x) mine |= (uint32_t)(row_seq[i] < 0 || row_seq[i] >= B);
  if (swa_start && swa_len)
    for (int64_t i = threadIdx.x; i < n_win; i += blockDim.x) {
      const int32_t st = swa_start[i], ln = swa_len[i];
      mine |= (uint32_t)(st < 0 || ln < 0 || ln > kWindowMax || (int64_t)st + ln > S);
    }
  if (idx)
    for (int64_t i = threadIdx.x; i < n_idx; i += blockDim.x) mine |= (uint32_t)(idx[i] < -1 || idx[i] >= T);
  if (mine) atomicOr(&bad, 1u);
  __syncthreads();
  if (threadIdx.x == 0) *out = bad;
}

static bool debug_enabled() {
  const char* e = getenv("CSA2_DEBUG");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

csa2_status debug_check(const int32_t* row_seq, int32_t R, int32_t B, const int32_t* swa_start,
                        const int32_t* swa_len, int64_t n_win, int32_t S, const int32_t* idx, int64_t n_idx,
                        int64_t T, hipStream_t s) {
  if (!debug_enabled() || (!row_seq && !(swa_start && swa_len) && !idx)) return CSA2_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ELAUNCH;
  uint32_t* out = dbg_bad_dev[dev].load(std::memory_order_acquire);
  if (!out) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_bad)) != hipSuccess || !p) return CSA2_ELAUNCH;
    out = static_cast<uint32_t*>(p);
    dbg_bad_dev[dev].store(out, std::memory_order_release);
  }
  debug_check_kernel<<<1, 256, 0, s>>>(row_seq, R, B, swa_start, swa_len, n_win, S, idx, n_idx, T, out);
  if (hipGetLastError() != hipSuccess) return CSA2_ELAUNCH;
  uint32_t host = 0u;
  if (hipMemcpyAsync(&host, out, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess) return CSA2_ELAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return CSA2_ELAUNCH;
  return host ? CSA2_EINVAL : CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" int32_t csa2_abi_version(void) { return 1; }

extern "C" const char* csa2_status_str(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument (null pointer, non-positive size or bad value)";
    case CSA2_ESHAPE: return "unsupported shape";
    case CSA2_EALIGN: return "pointer or stride not aligned as required";
    case CSA2_EWORKSPACE: return "workspace missing or too small";
    case CSA2_ELAUNCH: return "kernel launch failed";
    case CSA2_ESCRATCH: return "shape needs more than the fixed scratch array of the allocation-free call";
    default: return "unknown status";
  }
}
