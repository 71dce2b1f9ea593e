// Launchers shared between the library's translation units (not part of the C ABI).
#pragma once

#include "common.hpp"

namespace csa2 {

// Streaming pool selection.  The Full scan splits each row into blocks of 128
// positions (block b: positions [128 b, 128 b + 128)) and, for every visible
// score whose order-preserving key reaches the row's threshold tau_s, stores
// the pair (key, position) at kp [r][128 b + i] in position order, with the
// count of block b in cnt [r][b]; it also counts each candidate's digit
// min((key - tau_s) >> sh, 4095) in hist [r][0 .. 4096).  hist [r][4096 .. 8192)
// is the selection's second histogram (the top 12 bits of every visible key,
// filled only when a row is rebuilt).
constexpr int kBlockPositions = 128;
constexpr int kStreamBins = 4096;
constexpr int kStreamHistWords = 2 * kStreamBins;   // per row

struct StreamRow {
  uint32_t tau_s;       // candidate threshold; 0 = every visible position
  uint32_t sh;          // digit shift of the candidate histogram
  uint32_t n_list[2];   // entries in each selection's boundary-bin list
  uint32_t ticket;      // gather workgroups finished
  uint32_t mode;        // 0: candidates from the blocks; 1: from the scores row
  uint32_t pad0[2];
  uint32_t tau[2];      // each selection's k-th key
  uint32_t need_eq[2];  // keys equal to tau it takes, lowest positions first
  uint32_t k_eff[2];    // entries it writes
  uint32_t pad1[2];
};

struct CandOut {
  StreamRow* row;
  uint32_t* hist;       // [R][kStreamHistWords], zero before the scan
  uint2* kp;            // [R][T] (key, position)
  uint32_t* cnt;        // [R][n_blocks]
  int64_t n_blocks;     // blocks per row the scan writes counts for (4 per 512-position unit)
  const uint32_t* samp; // [R][index_sample_words()] sample keys: the scan derives each row's tau_s and sh
                        // from them (and stores them in the row state); null: already in the row state
  int32_t k;            // the selection size the threshold is taken for (with samp)
};

// Full-mode index scan on `s`; with cand, also emits the candidates (and then
// scores may be null: no scores are written).
void launch_index_scan(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T, const int32_t* row_seq,
                       const int64_t* row_limit, float* scores, const CandOut* cand, hipStream_t s,
                       const PageMap& pm);

// Query-block form of the candidate scan (chunked prefill: runs of query rows
// of one sequence share every key tile): candidates in blocks of bsz
// positions (a multiple of 128), kp [r][bsz b + i] and cnt [r][b] as above for
// all cand.n_blocks = ceil(T / bsz) blocks of every row; hist is not touched
// (a pass over the blocks builds it).  scores, if given, receives every score.
constexpr int kQueryBlockPositions = 1024;
void launch_index_block_cand(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T,
                             const int32_t* row_seq, const int64_t* row_limit, float* scores, const CandOut& cand,
                             int bsz, hipStream_t s, const PageMap& pm);

// a strided sample of each row's scores (samp: [R][index_sample_words()]
// scratch), with the rows' histogram and state cleared; with tau, also the
// threshold kernel that derives tau_s and the digit shift for a selection of
// k from the sample (without it the candidate scan derives them itself)
void launch_index_sample_tau(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int64_t T,
                             const int32_t* row_seq, const int64_t* row_limit, int32_t k, StreamRow* rows,
                             uint32_t* hist, uint32_t* samp, bool tau, hipStream_t s, const PageMap& pm);

// whether the candidate scan of R rows gives every workgroup a single row, so
// that it can take the row's threshold from the sample itself (CandOut::samp)
bool index_scan_derives_tau(int32_t R);
int64_t index_sample_words();

// blocks per row whose counts the candidate scan writes
int64_t index_scan_blocks(int64_t T);

// page-table arguments of the paged entry points: a table, a page size that is a
// multiple of kPageQuantum positions, and room for T positions
constexpr int32_t kPageQuantum = 128;
csa2_status check_pages(const int32_t* block_table, int64_t max_blocks, int32_t page, int64_t T);

// whether csa2_index_full uses the streaming scan (decode) rather than the
// query-block kernel (chunked prefill) for this row layout
bool index_scan_streams(int32_t R, const int32_t* row_seq);

// Opt-in validation (the environment variable CSA2_DEBUG set to anything but
// "0", read at every call): before its own launches a call checks its
// device-side row_seq entries against [0, B) (an entry outside reads another
// sequence's memory or past the arrays) and, strictly, the entries the kernels
// would otherwise skip: window bounds outside 0 <= start, 0 <= len <= 128,
// start + len <= S, and attention indices outside [-1, T).  It waits for the
// check on the stream and returns CSA2_EINVAL on a bad entry, launching nothing
// else.  Off: returns CSA2_OK at once.  (With it on, a call synchronises: not
// for graph capture.)
csa2_status debug_check(const int32_t* row_seq, int32_t R, int32_t B, const int32_t* swa_start,
                        const int32_t* swa_len, int64_t n_win, int32_t S, const int32_t* idx, int64_t n_idx,
                        int64_t T, hipStream_t s);

}  // namespace csa2
