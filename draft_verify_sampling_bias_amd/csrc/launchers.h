// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dspark.h"

namespace dspark {

// One launch of the fused Markov-bias + softmax-statistics tile kernel.
//   draft mode:    request n uses prev = prev_base[n * prev_stride] and the
//                  base-logit row U_base + n * U_stride; writes per (n, tile)
//                  the max / lowest argmax of s = U + B and, for sampled
//                  requests, the four 32-row sums of exp((s - max)/T).
//   residual mode: request n takes (flag, prev, U row, target row) from
//                  rs_info and (Mq, Zq, Mp, Zp) from rs_stats and writes the
//                  four 32-row sums of max(0, p - q); flag 0 => skipped.
struct TileParams {
  const void* W1;
  const void* W2;
  int V, rank, R, n_tiles;
  const int32_t* prev_base;
  int prev_stride;
  const float* U_base;
  int64_t U_stride;
  const float* temp;
  const int32_t* rs_info;
  const float* rs_stats;
  const float* U;        // [R * gamma, V] (residual mode)
  const float* target;   // [n_rows, V]   (residual mode)
  float* part;           // [R][n_tiles][kPartFloats]
};

// Per-position draft finish: turns the tile records into y / q_tok / q_stats.
struct FinishParams {
  const float* part;
  int n_tiles, V, rank, R, gamma, k;
  const void* W1;
  const void* W2;
  const int32_t* prev_base;
  int prev_stride;
  const float* U_base;
  int64_t U_stride;
  const float* temp;
  const float* u_draft;
  int32_t* y;
  float* q_tok;
  float* q_stats;
};

struct VerifyParams {
  int R, gamma, V, rank, n_chunks, n_tiles;
  int64_t n_rows;
  const float* target;
  const int32_t* row_offsets;
  const float* U;
  const void* W1;
  const void* W2;
  const int32_t* anchor;
  const float* temp;
  const int32_t* y;
  const float* q_tok;
  const float* q_stats;
  const float* u_accept;
  const float* u_final;
  int32_t* n_accept;
  int32_t* out_tok;
  float* p_tok;
  float* vpart;      // [n_rows][n_chunks][kChunkFloats]
  int32_t* rs_info;  // [R][4]
  float* rs_stats;   // [R][4]
  float* rpart;      // [R][n_tiles][kPartFloats]
};

hipError_t launch_bias_tile(const TileParams& p, int wdtype, bool residual, hipStream_t s);
hipError_t launch_draft_finish(const FinishParams& p, int wdtype, hipStream_t s);
hipError_t launch_verify_stats(const VerifyParams& p, hipStream_t s);
hipError_t launch_verify_finish(const VerifyParams& p, hipStream_t s);
hipError_t launch_residual_finish(const VerifyParams& p, int wdtype, hipStream_t s);
hipError_t launch_schedule(const dspark_schedule_args& a, hipStream_t s);

}  // namespace dspark
