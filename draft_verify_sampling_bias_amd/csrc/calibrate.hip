// Sequential temperature scaling of the confidence head ("DSpark" explainer
// section 8: a confidence that ranks well but is over-confident in absolute
// value makes wrong capacity decisions, so the cumulative probabilities are
// corrected by a posterior temperature calibration, position by position
// from left to right).
//
// Fit: one workgroup of 1024 threads per block position k.  Calibration
// block i reached k iff n_acc[i] >= k and was accepted there iff
// n_acc[i] > k.  The inverse temperature beta_k is the maximum-likelihood
// one of P(accept | reached) = sigmoid(beta z): the root of the score
//   g(beta) = sum over reached i of z_ik (sigmoid(beta z_ik) - y_ik),
// which is non-decreasing in beta, found by bisection on [2^-8, 2^8] in fp64
// (an end of the interval when g has no sign change there; beta = 1 when no
// block reached k or all its logits are 0).  Each evaluation of g is a
// block-wide fp64 sum; every thread reads the same wavefront totals in the
// same order, so the bisection decisions are uniform.  Up to 8192 blocks
// the thread's values stay in registers, beyond that they are re-read each
// evaluation (from L2 after the first).
//
// Apply: c[r, k] = sigmoid(z[r, k] / tau[k]) in fp64, rounded once to fp32.
// Logits are clamped to [-64, 64], NaN -> 0, on both paths.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kFitThreads = 1024;
constexpr int kFitRegs = 8;  // blocks per thread held in registers
constexpr double kBetaMin = 0.00390625, kBetaMax = 256.0;
constexpr int kMaxBisect = 100;

__device__ __forceinline__ float clamp_logit(float z) {
  return (z != z) ? 0.0f : fminf(fmaxf(z, -64.0f), 64.0f);
}

__device__ __forceinline__ double sigmoid64(double x) { return 1.0 / (1.0 + exp(-x)); }

// one calibration block at position k: its clamped logit and outcome code
// (0 = did not reach k, 1 = reached and rejected, 2 = reached and accepted)
__device__ __forceinline__ void fit_item(const dspark_sts_fit_args& a, int i, int k, float& z, int& code) {
  const int n = min(max(a.n_acc[i], 0), a.gamma);
  z = clamp_logit(a.z[static_cast<int64_t>(i) * a.gamma + k]);
  code = (n < k) ? 0 : (n > k ? 2 : 1);
}

__device__ __forceinline__ double score_term(double beta, float z, int code) {
  const double zd = static_cast<double>(z);
  const double y = (code == 2) ? 1.0 : 0.0;
  return (code == 0) ? 0.0 : zd * (sigmoid64(beta * zd) - y);
}

__device__ __forceinline__ double wave_sum64(double x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

template <bool CACHED>
__global__ void __launch_bounds__(kFitThreads) sts_fit_kernel(dspark_sts_fit_args a) {
  // two slots per wavefront, alternating between evaluations, so one barrier
  // per evaluation suffices
  __shared__ double part[2][16];
  __shared__ int s_cnt[16], s_nz[16];
  const int k = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;

  float zr[CACHED ? kFitRegs : 1];
  int cr[CACHED ? kFitRegs : 1];
  int reached = 0, nonzero = 0;
  if (CACHED) {
#pragma unroll
    for (int j = 0; j < kFitRegs; ++j) {
      const int i = tid + j * kFitThreads;
      zr[j] = 0.0f;
      cr[j] = 0;
      if (i < N) fit_item(a, i, k, zr[j], cr[j]);
      reached += cr[j] != 0;
      nonzero |= (cr[j] != 0) & (zr[j] != 0.0f);
    }
  } else {
    for (int i = tid; i < N; i += kFitThreads) {
      float z;
      int code;
      fit_item(a, i, k, z, code);
      reached += code != 0;
      nonzero |= (code != 0) & (z != 0.0f);
    }
  }
  // block totals of the reached count and of "some reached logit is nonzero"
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    reached += __shfl_xor(reached, d);
    nonzero |= __shfl_xor(nonzero, d);
  }
  if (lane == 0) {
    s_cnt[wave] = reached;
    s_nz[wave] = nonzero;
  }
  __syncthreads();
  int any_info = 0;
  for (int w = 0; w < 16; ++w) any_info |= s_nz[w];

  // g(beta), block-wide; slot alternates between calls
  int slot = 0;
  auto score = [&](double beta) -> double {
    double t = 0.0;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < kFitRegs; ++j) t += score_term(beta, zr[j], cr[j]);
    } else {
      for (int i = tid; i < N; i += kFitThreads) {
        float z;
        int code;
        fit_item(a, i, k, z, code);
        t += score_term(beta, z, code);
      }
    }
    t = wave_sum64(t);
    if (lane == 0) part[slot][wave] = t;
    __syncthreads();
    double g = 0.0;
    for (int w = 0; w < 16; ++w) g += part[slot][w];
    slot ^= 1;
    return g;
  };

  double beta = 1.0;
  if (any_info) {
    const double g_lo = score(kBetaMin);
    const double g_hi = score(kBetaMax);
    if (g_lo >= 0.0) {
      beta = kBetaMin;
    } else if (g_hi <= 0.0) {
      beta = kBetaMax;
    } else {
      double lo = kBetaMin, hi = kBetaMax;  // g(lo) < 0 < g(hi)
      for (int it = 0; it < kMaxBisect; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;  // adjacent doubles (uniform)
        if (score(mid) > 0.0) hi = mid;
        else lo = mid;
      }
      beta = 0.5 * (lo + hi);
    }
  }
  if (tid == 0) a.tau[k] = static_cast<float>(1.0 / beta);
}

__global__ void __launch_bounds__(256) sts_apply_kernel(dspark_sts_apply_args a) {
  const int64_t n = static_cast<int64_t>(a.R) * a.gamma;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int k = static_cast<int>(i % a.gamma);
    const double x = static_cast<double>(clamp_logit(a.z[i])) / static_cast<double>(a.tau[k]);
    a.c[i] = static_cast<float>(sigmoid64(x));
  }
}

}  // namespace

hipError_t launch_sts_fit(const dspark_sts_fit_args& a, hipStream_t s) {
  if (a.N <= kFitRegs * kFitThreads)
    hipLaunchKernelGGL(sts_fit_kernel<true>, dim3(a.gamma), dim3(kFitThreads), 0, s, a);
  else
    hipLaunchKernelGGL(sts_fit_kernel<false>, dim3(a.gamma), dim3(kFitThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sts_apply(const dspark_sts_apply_args& a, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.R) * a.gamma;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(sts_apply_kernel, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace dspark
