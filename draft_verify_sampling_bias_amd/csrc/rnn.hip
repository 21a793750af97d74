// State update of the RNN sequential head ("DSpark" explainer section 7: a
// sequential head that carries a longer in-block state than the Markov head;
// the pages give it no equations).  Reading: the Elman recurrence
//   h_k = act(A h_{k-1} + W1[prev_k]),  h_{-1} = 0,
// prev_0 = anchor, prev_k = y_{k-1}; the bias of position k is W2 h_k (the
// fused bias kernel reads h_k instead of W1[prev]).  With A = 0 and the
// identity activation this is exactly the Markov head.
//
// Workgroup (n, b) computes outputs j = 32 b .. 32 b + 31 of request n with
// eight lanes per output: lane p of an output's group takes the 16-byte
// pieces p, p + 8, p + 16, ... of row j of A (bf16, eight weights each; the
// eight lanes read 128 contiguous bytes per load, and all of a lane's loads
// are issued before the first is used), multiplies them with h_{k-1} (fp32,
// in LDS) in fp32 in index order, and the eight partial sums are added by a
// fixed shuffle tree; then W1[prev, j] is added and the activation applied.
// The state is stored as a double-bf16 value: hi = bf16(h), lo = bf16(h -
// hi), h = hi + lo.  The fused bias kernel splits it into the same two bf16
// planes for its matrix-core products, so every consumer of the state (that
// kernel, the finish rescans, the verify's residual, the next state) sees
// the same number.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kRnnThreads = 256;
constexpr int kLanesPerOut = 8;
constexpr int kOutsPerGroup = kRnnThreads / kLanesPerOut;               // 32
constexpr int kMaxPieces = DSPARK_MAX_RANK / 8 / kLanesPerOut;          // 8 per lane

__global__ void __launch_bounds__(kRnnThreads) rnn_state_kernel(RnnStateParams p) {
  __shared__ __attribute__((aligned(16))) float hp[DSPARK_MAX_RANK];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int rank = p.rank, V = p.V;
  const int lp = tid & (kLanesPerOut - 1);
  const int j = blockIdx.y * kOutsPerGroup + tid / kLanesPerOut;
  const int jc = min(j, rank - 1);
  const int64_t row = static_cast<int64_t>(n) * p.gamma + p.k;
  const int prev = clampi(p.k == 0 ? p.anchor[n] : p.y[row - 1], 0, V - 1);
  const float w1 = bf16_to_f32(p.W1[static_cast<int64_t>(prev) * rank + jc]);
  float z = 0.0f;
  if (p.k > 0) {  // grid-uniform
    const int G = rank / 8;  // 16-byte pieces per row of A
    const uint16_t* a = p.A + static_cast<int64_t>(jc) * rank;
    u32x4_t w[kMaxPieces];
#pragma unroll
    for (int q = 0; q < kMaxPieces; ++q) {
      const int pc = min(q * kLanesPerOut + lp, G - 1);
      w[q] = *reinterpret_cast<const u32x4_t*>(a + pc * 8);
    }
    for (int i = tid; i < rank; i += kRnnThreads) hp[i] = p.h[(row - 1) * rank + i];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxPieces; ++q) {
      const int pc = q * kLanesPerOut + lp;
      if (pc < G) {
        const f32x4_t h0 = *reinterpret_cast<const f32x4_t*>(hp + pc * 8);
        const f32x4_t h1 = *reinterpret_cast<const f32x4_t*>(hp + pc * 8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = e < 2 ? h0[2 * e] : h1[2 * e - 4];
          const float x1 = e < 2 ? h0[2 * e + 1] : h1[2 * e - 3];
          z = fmaf(__uint_as_float(w[q][e] << 16), x0, z);
          z = fmaf(__uint_as_float(w[q][e] & 0xffff0000u), x1, z);
        }
      }
    }
    // the eight partial sums of an output, in a fixed tree
#pragma unroll
    for (int off = kLanesPerOut / 2; off > 0; off >>= 1) z += __shfl_xor(z, off, kLanesPerOut);
  }
  if (lp == 0 && j < rank) p.h[row * rank + j] = double_bf16(rnn_act(z + w1, p.act));
}

}  // namespace

hipError_t launch_rnn_state(const RnnStateParams& p, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.R), static_cast<unsigned>((p.rank + kOutsPerGroup - 1) / kOutsPerGroup));
  hipLaunchKernelGGL(rnn_state_kernel, grid, dim3(kRnnThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
