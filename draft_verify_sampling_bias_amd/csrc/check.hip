// Device input checks of the DSPARK_CHECK_INPUTS flag (debug).
//
// One workgroup inspects the small device inputs of a call (token ids,
// uniforms, confidences, verify row offsets) and writes the DSPARK_BAD_*
// bits it found into the error word at the start of the call's workspace.
// The llama.cpp PR #25173 review asks that a non-uniform block never be
// inferred silently and that a degraded result never be silent; the hot
// kernels clamp such values so that no access leaves its buffer, and this
// pass is how a caller learns that it happened.  Reads only; the word is
// written once, by one thread, after the whole workgroup has looked.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kCheckThreads = 1024;

__global__ void __launch_bounds__(kCheckThreads) input_check_kernel(CheckParams p) {
  __shared__ uint32_t s_bits;
  const int tid = threadIdx.x;
  if (tid == 0) s_bits = 0u;
  __syncthreads();
  uint32_t bits = 0u;
  for (int a = 0; a < kCheckMaxArrays; ++a) {
    const int32_t* ids = p.ids[a];
    if (ids == nullptr) continue;
    for (int64_t i = tid; i < p.n_ids[a]; i += kCheckThreads) {
      const int32_t v = ids[i];
      if (v < 0 || v >= p.V) bits |= DSPARK_BAD_TOKEN;
    }
  }
  for (int a = 0; a < kCheckMaxArrays; ++a) {
    const float* u = p.unif[a];
    if (u == nullptr) continue;
    for (int64_t i = tid; i < p.n_unif[a]; i += kCheckThreads) {
      const float x = u[i];
      if (!(x >= 0.0f && x < 1.0f)) bits |= DSPARK_BAD_UNIFORM;  // NaN fails both
    }
  }
  if (p.conf != nullptr) {
    for (int64_t i = tid; i < p.n_conf; i += kCheckThreads) {
      const float x = p.conf[i];
      if (!(x >= 0.0f && x <= 1.0f)) bits |= DSPARK_BAD_CONFIDENCE;
    }
  }
  if (p.offsets != nullptr) {
    // request r owns rows offsets[r] .. offsets[r + 1] - 1: between 1 and
    // gamma + 1 of them (verify length l = rows - 1 in [0, gamma]), and the
    // rows stay inside [0, n_rows]
    for (int r = tid; r < p.R; r += kCheckThreads) {
      const int64_t lo = p.offsets[r], hi = p.offsets[r + 1];
      const int64_t rows = hi - lo;
      if (rows < 1 || rows > static_cast<int64_t>(p.gamma) + 1 || lo < 0 || hi > p.n_rows)
        bits |= DSPARK_BAD_LENGTH;
    }
  }
  if (bits != 0u) atomicOr(&s_bits, bits);
  __syncthreads();
  if (tid == 0) *p.err = s_bits;
}

}  // namespace

hipError_t launch_input_check(const CheckParams& p, hipStream_t s) {
  if (p.err == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(input_check_kernel, dim3(1), dim3(kCheckThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
