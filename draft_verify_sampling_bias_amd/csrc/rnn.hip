// State update of the RNN sequential head ("DSpark" explainer section 7: a
// sequential head that carries a longer in-block state than the Markov head;
// the pages give it no equations).  Reading: the Elman recurrence
//   h_k = act(A h_{k-1} + W1[prev_k]),  h_{-1} = 0,
// prev_0 = anchor, prev_k = y_{k-1}; the bias of position k is W2 h_k (the
// fused bias kernel reads h_k instead of W1[prev]).  With A = 0 and the
// identity activation this is exactly the Markov head.
//
// Workgroup (n, b) is one wavefront computing outputs j = 64 b + lane of
// request n: the dot product of row j of A (bf16, eight weights per 16-byte
// load, the loads of a row issued together) with h_{k-1} (fp32, in LDS,
// read as broadcasts), accumulated in fp32 in index order, plus W1[prev, j],
// then the activation.  The state is stored as a double-bf16 value: hi =
// bf16(h), lo = bf16(h - hi), h = hi + lo.  The fused bias kernel splits it
// into the same two bf16 planes for its matrix-core products, so every
// consumer of the state (that kernel, the finish rescans, the verify's
// residual, the next state) sees the same number.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kRnnThreads = 64;

__device__ __forceinline__ float rnn_act(float z, int act) { return act == DSPARK_ACT_TANH ? tanhf(z) : z; }

// h rounded to the nearest double-bf16 value (16 significant bits)
__device__ __forceinline__ float double_bf16(float h) {
  const float hi = __uint_as_float(bf16_rne_bits(h) << 16);
  const float lo = __uint_as_float(bf16_rne_bits(h - hi) << 16);
  return hi + lo;
}

__global__ void __launch_bounds__(kRnnThreads) rnn_state_kernel(RnnStateParams p) {
  __shared__ float hp[DSPARK_MAX_RANK];
  const int n = blockIdx.x, lane = threadIdx.x;
  const int rank = p.rank, V = p.V;
  const int j = blockIdx.y * kRnnThreads + lane;
  const int64_t row = static_cast<int64_t>(n) * p.gamma + p.k;
  const int prev = clampi(p.k == 0 ? p.anchor[n] : p.y[row - 1], 0, V - 1);
  const float w1 = bf16_to_f32(p.W1[static_cast<int64_t>(prev) * rank + min(j, rank - 1)]);
  float z = 0.0f;
  if (p.k > 0) {  // grid-uniform
    for (int i = lane; i < rank; i += kRnnThreads) hp[i] = p.h[(row - 1) * rank + i];
    __syncthreads();
    const uint16_t* a = p.A + static_cast<int64_t>(min(j, rank - 1)) * rank;
#pragma unroll 8
    for (int i = 0; i < rank; i += 8) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(a + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        z = fmaf(__uint_as_float(w[q] << 16), hp[i + 2 * q], z);
        z = fmaf(__uint_as_float(w[q] & 0xffff0000u), hp[i + 2 * q + 1], z);
      }
    }
  }
  if (j < rank) p.h[row * rank + j] = double_bf16(rnn_act(z + w1, p.act));
}

}  // namespace

hipError_t launch_rnn_state(const RnnStateParams& p, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.R), static_cast<unsigned>((p.rank + kRnnThreads - 1) / kRnnThreads));
  hipLaunchKernelGGL(rnn_state_kernel, grid, dim3(kRnnThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
