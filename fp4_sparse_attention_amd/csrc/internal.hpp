// Launchers shared between the library's translation units (not part of the C ABI).
#pragma once

#include "common.hpp"

namespace csa2 {

// Full-mode index scan on `s`; with top_hist (uint32 [R][4096], zeroed), also
// counts the top 12 bits of every visible score's order-preserving key.
void launch_index_scan(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T, const int32_t* row_seq,
                       const int64_t* row_limit, float* scores, uint32_t* top_hist, hipStream_t s);

// whether csa2_index_full uses the streaming scan (decode) rather than the
// query-block kernel (chunked prefill) for this row layout
bool index_scan_streams(int32_t R, const int32_t* row_seq);

}  // namespace csa2
