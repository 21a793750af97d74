// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dspark.h"

namespace dspark {

// A request that rejected a sampled draft, as handed from verify_finish to
// the residual pass of the 64-row path (which visits only these requests).
struct ResidualEntry {
  int32_t n, prev, urow, trow;   // request, previous token, U row, target row
  float Mq, Zq, Mp, Zp;          // softmax statistics of q and p at that position
  float T;                       // temperature
  float pad[3];
};
static_assert(sizeof(ResidualEntry) == 48, "ResidualEntry layout");

// One launch of the fused Markov-bias + softmax-statistics kernel.
//   draft mode:    request n uses prev = prev_base[n * prev_stride] and the
//                  base-logit row U_base + n * U_stride; writes per (n, segment)
//                  the record (max of s = U + B, sum of exp((s - max)/T)) for a
//                  sampled request or (max, lowest argmax) for a greedy one.
//   residual mode: request n takes (flag, prev, U row, target row) from
//                  rs_info and (Mq, Zq, Mp, Zp) from rs_stats and writes
//                  (0, sum of max(0, p - q)) per segment; flag 0 => skipped.
//                  The 64-row path visits only the rs_count[0] entries of
//                  rs_list instead.
struct TileParams {
  const void* W1;
  const void* W2;
  int V, rank, R;
  int seg_rows, n_seg;
  const int32_t* prev_base;
  int prev_stride;
  const float* U_base;
  int64_t U_stride;
  const float* temp;
  const int32_t* rs_info;
  const float* rs_stats;
  const int32_t* rs_count;          // 64-row path, residual mode
  const ResidualEntry* rs_list;
  const float* U;        // [u_rows = R * gamma, V] (residual mode)
  const float* target;   // [t_rows = n_rows, V]    (residual mode)
  int64_t u_rows, t_rows;
  float* part;           // [record_rows][n_seg][kRecFloats] segment records
  // 16-row path: when set, the W2 fragments are read from this
  // fragment-packed copy (dspark_pack_w2) instead of W2
  const uint16_t* w2p;
  // RNN head (16-row path), else null: H is the fp32 state instead of
  // W1[prev]; draft mode: request n's row at h_base + n * h_stride;
  // residual mode: row urow (U row index n * gamma + position) of h_base
  const float* h_base;
  int64_t h_stride;
  // RNN head, draft mode: when n_seg_a > 0 the walk also covers n_seg_a =
  // ceil(rank / 16) segments of the recurrence matrix A (rank x rank, bf16)
  // after the n_seg vocabulary segments, read from A (row-major, like W2)
  // or, when w2p is set, from its fragment-packed copy ap; for them it
  // stores z = A h of request n (fp32, rank values) at z_out + n * h_stride
  // instead of records
  int n_seg_a;
  const uint16_t* A;
  const uint16_t* ap;
  float* z_out;
};

// Per-position draft finish: turns the segment records into y / q_tok / q_stats.
struct FinishParams {
  const float* part;     // segment records of the fused bias kernel
  int seg_rows, n_seg, V, rank, R, gamma, k;
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
  // RNN head, else null: h for (n, k) is the fp32 row hstate + (n * gamma + k)
  // * rank instead of W1[prev]
  float* hstate;
  // RNN head with the next state fused into this finish (else null): the
  // fused bias kernel stored z = A h in the state row of (n, k + 1); the
  // finish of (n, k < gamma - 1) turns it into act(z + W1[y]) with this
  // activation (A itself is not read here)
  const uint16_t* A;
  int act;
  // when set, block 0 writes 0 to this error word (a call made without the
  // input checks still rewrites the word of its workspace)
  uint32_t* err_clear;
};

struct VerifyParams {
  int R, gamma, V, rank, n_chunks, seg_rows, n_seg;
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
  float* rpart;      // [record_rows][n_seg][kRecFloats] residual segment records
  // 64-row path (else null): verify_stats zeroes the count, verify_finish
  // appends every request that needs the residual pass
  int32_t* rs_count;
  ResidualEntry* rs_list;  // [R]
  // RNN head, else null: the draft's fp32 states [R * gamma, rank]; the
  // residual of request n at position j uses row n * gamma + j
  const float* hstate;
  // when set, verify_stats writes 0 to this error word (as FinishParams)
  uint32_t* err_clear;
};

// The device input checks of one call (DSPARK_CHECK_INPUTS): token arrays
// must hold ids in [0, V), uniform arrays values in [0, 1), the confidence
// values in [0, 1], and the verify row offsets 1 .. gamma + 1 rows per
// request inside [0, n_rows].  Unused entries are NULL.  The bits found are
// written to *err (the first word of the call's workspace).
constexpr int kCheckMaxArrays = 2;
struct CheckParams {
  uint32_t* err;
  const int32_t* ids[kCheckMaxArrays];
  int64_t n_ids[kCheckMaxArrays];
  int V;
  const float* unif[kCheckMaxArrays];
  int64_t n_unif[kCheckMaxArrays];
  const float* conf;
  int64_t n_conf;
  const int32_t* offsets;  // [R + 1]
  int R, gamma;
  int64_t n_rows;
};
hipError_t launch_input_check(const CheckParams& p, hipStream_t s);

// ev0 / ev1 (optional): events attached to the kernel's dispatch, recorded
// when it starts and when it ends.
hipError_t launch_bias_tile(const TileParams& p, int wdtype, bool residual, int num_cu, hipStream_t s,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_draft_finish(const FinishParams& p, int wdtype, hipStream_t s);
// whether launch_draft_finish takes the finish that can fuse the RNN head's
// next state (p.A)
bool draft_finish_fuses_state(const FinishParams& p, int wdtype);

// The RNN head's state of position k for every request:
// h[n, k] = act(A h[n, k-1] + W1[prev]) (h[n, -1] = 0), fp32.
struct RnnStateParams {
  int R, gamma, V, rank, k, act;
  const uint16_t* W1;      // [V, rank] bf16
  const uint16_t* A;       // [rank, rank] bf16
  const int32_t* anchor;   // [R]
  const int32_t* y;        // [R, gamma] (prev of k > 0)
  float* h;                // [R, gamma, rank]: row k - 1 read, row k written
};
hipError_t launch_rnn_state(const RnnStateParams& p, hipStream_t s);
hipError_t launch_verify_stats(const VerifyParams& p, hipStream_t s);
hipError_t launch_verify_finish(const VerifyParams& p, hipStream_t s);
hipError_t launch_residual_finish(const VerifyParams& p, int wdtype, hipStream_t s);
hipError_t launch_schedule(const dspark_schedule_args& a, hipStream_t s);
hipError_t launch_pack_w2(const dspark_pack_w2_args& a, hipStream_t s);
// the static confidence cutoff; a.K is not read
hipError_t launch_schedule_cutoff(const dspark_schedule_args& a, float conf_min, hipStream_t s);
// the hardware-aware capacity (one workgroup)
hipError_t launch_capacity(const dspark_capacity_args& a, hipStream_t s);
// sequential temperature scaling: the fit (one workgroup per position) and
// the calibrated confidence
hipError_t launch_sts_fit(const dspark_sts_fit_args& a, hipStream_t s);
hipError_t launch_sts_apply(const dspark_sts_apply_args& a, hipStream_t s);

}  // namespace dspark
