// Host-side argument checks and workspace layout for libdspark.
// Pure C++17 (no HIP): also compiled on its own for host-only tests.
#pragma once

#include <cstddef>
#include <cstdint>

#include "dspark.h"

namespace dspark {

// Vocabulary rows per workgroup of the fused bias + softmax kernels
// (4 wavefronts x one 32-row MFMA tile each).
constexpr int kTileRows = 128;
constexpr int kSubRows = 32;                 // rows per wavefront sub-tile
constexpr int kPartFloats = 8;               // floats per (request, tile) record
// Target-row elements per workgroup of the verify statistics kernel.
constexpr int kChunk = 4096;
constexpr int kChunkFloats = 4;              // floats per (row, chunk) record
constexpr std::size_t kWsAlign = 256;

struct DraftPlan {
  int n_tiles = 0;
  std::size_t part_off = 0;   // [R][n_tiles][kPartFloats] float
  std::size_t total = 0;
};

struct VerifyPlan {
  int n_tiles = 0;
  int n_chunks = 0;
  std::size_t vpart_off = 0;    // [n_rows][n_chunks][kChunkFloats] float
  std::size_t rsinfo_off = 0;   // [R][4] int32: flag, prev, U row, target row
  std::size_t rsstats_off = 0;  // [R][4] float: Mq, 1/Zq, Mp, 1/Zp
  std::size_t rpart_off = 0;    // [R][n_tiles][kPartFloats] float
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
