// Host-side argument checks and workspace layout for libdspark.
// Pure C++17 (no HIP): also compiled on its own for host-only tests.
#pragma once

#include <cstddef>
#include <cstdint>

#include "dspark.h"

namespace dspark {

// The fused bias + softmax kernels reduce each request's logits over
// vocabulary segments of 16 rows (bf16 weights, R <= 64: one 16x16x32 MFMA
// row block per wavefront) or 32 rows (otherwise: 32x32 MFMA row blocks) to
// one record of two floats per (request, segment).
constexpr int kSegSmall = 16;
constexpr int kSegLarge = 32;
constexpr int kSmallMaxR = 64;               // requests held by the 16-row path
constexpr int kRecFloats = 2;                // floats per (request, segment) record
// Record arrays of the 16-row path hold kSmallMaxR request rows whatever R
// is: every lane of the kernel stores its record unconditionally (rows of
// absent requests are padding and never read), which keeps divergent
// branches out of the kernel's streaming loop.
inline int record_rows(int seg_rows, int R) { return seg_rows == kSegSmall ? kSmallMaxR : R; }

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

// Rows per segment for a batch of R requests with weights of type wdtype.
inline int seg_rows_for(int32_t R, int32_t wdtype) {
  return (wdtype == DSPARK_W_BF16 && R <= kSmallMaxR) ? kSegSmall : kSegLarge;
}

struct DraftPlan {
  int seg_rows = 0;
  int n_seg = 0;
  std::size_t part_off = 0;  // [record_rows][n_seg][kRecFloats] float
  std::size_t hbuf_off = 0;  // 16-row path: [kSmallMaxR][rank] bf16, W1 rows of the next prev tokens
  std::size_t total = 0;
};

struct VerifyPlan {
  int seg_rows = 0;
  int n_seg = 0;
  int n_chunks = 0;
  std::size_t vpart_off = 0;    // [n_rows][n_chunks][kChunkFloats] float
  std::size_t rsinfo_off = 0;   // [R][4] int32: flag, prev, U row, target row
  std::size_t rsstats_off = 0;  // [R][4] float: Mq, 1/Zq, Mp, 1/Zp
  std::size_t rpart_off = 0;    // [record_rows][n_seg][kRecFloats] float
  std::size_t total = 0;
};

// Size checks shared by draft and verify.  Returns a dspark_status.
int check_dims(int32_t R, int32_t gamma, int32_t V, int32_t rank, int32_t wdtype);

int plan_draft(const dspark_draft_args* a, DraftPlan* plan);      // sizes only
int validate_draft(const dspark_draft_args* a, DraftPlan* plan);  // sizes + pointers + workspace

int plan_verify(const dspark_verify_args* a, VerifyPlan* plan);
int validate_verify(const dspark_verify_args* a, VerifyPlan* plan);

int validate_schedule(const dspark_schedule_args* a);

int64_t schedule_rows(int32_t R, int32_t gamma, int64_t K);
const char* status_string(int status);

}  // namespace dspark
