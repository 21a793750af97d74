// Host-side argument checks and workspace layout for libdspark.
// Pure C++17 (no HIP): also compiled on its own for host-only tests.
#pragma once

#include <cstddef>
#include <cstdint>

#include "dspark.h"

namespace dspark {

// The fused bias + softmax kernels reduce each request's logits over
// vocabulary segments to one record of two floats per (request, segment):
//   16 rows  bf16 weights, R <= 64 (one 16x16x32 MFMA row block per wavefront)
//   64 rows  bf16 weights, R > 64 (four row blocks held by one wavefront)
//   32 rows  fp32 weights (32x32x2 MFMA row blocks)
constexpr int kSegSmall = 16;
constexpr int kSegLarge = 32;
constexpr int kSegWide = 64;
constexpr int kSmallMaxR = 64;               // requests held by the 16-row path
constexpr int kWideChunk = 16;               // requests per chunk of the 64-row path
constexpr int kRecFloats = 2;                // floats per (request, segment) record
// Record arrays hold more rows than requests where the kernels store
// unconditionally (which keeps divergent branches out of their streaming
// loops; the extra rows are never read):
//   16-row path: kSmallMaxR rows whatever R is;
//   64-row path: R + 16 rows catch the requests past R of the last chunk,
//                and row R + 16 the segments past the vocabulary of the
//                last workgroup.
constexpr int kWidePadRows = kWideChunk + 1;
inline int record_rows(int seg_rows, int R) {
  return seg_rows == kSegSmall ? kSmallMaxR : (seg_rows == kSegWide ? R + kWidePadRows : R);
}

#if defined(__HIPCC__)
#define DSPARK_HD __host__ __device__
#else
#define DSPARK_HD
#endif

// Balanced partition of n items into n_ranges contiguous ranges (the first
// n % n_ranges ranges one item longer): first item of range g.
DSPARK_HD inline int range_start(int g, int n, int n_ranges) {
  const int q = n / n_ranges, r = n % n_ranges;
  return g * q + (g < r ? g : r);
}
// Target-row elements per workgroup of the verify statistics kernel.
constexpr int kChunk = 4096;
constexpr int kChunkFloats = 4;              // floats per (row, chunk) record
constexpr std::size_t kWsAlign = 256;
// Every draft and verify workspace (and a schedule workspace, which exists
// only for the input checks) starts with a header holding the error word of
// the device input checks at byte 0.
constexpr std::size_t kHeaderBytes = DSPARK_WORKSPACE_HEADER;
static_assert(DSPARK_WORKSPACE_HEADER % 256 == 0, "header keeps the workspace 256-byte aligned");

// k-steps (32 ranks each) of the 16-row kernel for a rank: 2, 4, 8 or 16.
// The fragment-packed W2 layout uses the same count.
inline int seg16_ksteps(int rank) { return rank <= 64 ? 2 : (rank <= 128 ? 4 : (rank <= 256 ? 8 : 16)); }

// Fragment-packed W2 (bf16): for each 16-row segment s and k-step ks, the
// 64 lanes' 16-byte MFMA A fragments in lane order, 1 KiB contiguous; lane
// L = 16 kq + l holds W2[16 s + l][32 ks + 8 kq .. +8] (zero past V or rank).
inline std::size_t w2_packed_bytes(int V, int rank) {
  if (V < 1) return 0;
  return (static_cast<std::size_t>(V) + 15) / 16 * static_cast<std::size_t>(seg16_ksteps(rank)) * 1024;
}

// Rows per segment for a batch of R requests with weights of type wdtype.
inline int seg_rows_for(int32_t R, int32_t wdtype) {
  if (wdtype != DSPARK_W_BF16) return kSegLarge;
  return R <= kSmallMaxR ? kSegSmall : kSegWide;
}

struct DraftPlan {
  int seg_rows = 0;
  int n_seg = 0;
  std::size_t part_off = 0;  // [record_rows][n_seg][kRecFloats] float
  // RNN head on the 16-row path: the fragment-packed copy of A (rank rows,
  // w2_packed_bytes(rank, rank)), made by the call when W2_packed is given
  std::size_t ap_off = 0;
  std::size_t total = 0;
  bool check = false;        // DSPARK_CHECK_INPUTS
};

struct VerifyPlan {
  int seg_rows = 0;
  int n_seg = 0;
  int n_chunks = 0;
  std::size_t vpart_off = 0;    // [n_rows][n_chunks][kChunkFloats] float
  std::size_t rsinfo_off = 0;   // [R][4] int32: flag, prev, U row, target row
  std::size_t rsstats_off = 0;  // [R][4] float: Mq, 1/Zq, Mp, 1/Zp
  std::size_t rpart_off = 0;    // [record_rows][n_seg][kRecFloats] float
  // 64-row path: the requests that need the residual pass, compacted
  std::size_t rcount_off = 0;   // int32 count
  std::size_t rlist_off = 0;    // [R] ResidualEntry (48 bytes)
  std::size_t total = 0;
  bool check = false;           // DSPARK_CHECK_INPUTS
};

constexpr std::size_t kResidualEntryBytes = 48;

// Size checks shared by draft and verify.  Returns a dspark_status.
int check_dims(int32_t R, int32_t gamma, int32_t V, int32_t rank, int32_t wdtype);

int plan_draft(const dspark_draft_args* a, DraftPlan* plan);      // sizes only
int validate_draft(const dspark_draft_args* a, DraftPlan* plan);  // sizes + pointers + workspace

int plan_verify(const dspark_verify_args* a, VerifyPlan* plan);
int validate_verify(const dspark_verify_args* a, VerifyPlan* plan);

// Schedule calls: workspace bytes (the header with DSPARK_CHECK_INPUTS, else 0).
int plan_schedule(const dspark_schedule_args* a, std::size_t* bytes);
int plan_cutoff(const dspark_cutoff_args* a, std::size_t* bytes);
int validate_schedule(const dspark_schedule_args* a);
int validate_cutoff(const dspark_cutoff_args* a);
int validate_pack_w2(const dspark_pack_w2_args* a);
int validate_capacity(const dspark_capacity_args* a);
int validate_sts_fit(const dspark_sts_fit_args* a);
int validate_sts_apply(const dspark_sts_apply_args* a);

int64_t schedule_rows(int32_t R, int32_t gamma, int64_t K);
const char* status_string(int status);

}  // namespace dspark
