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
// which is non-decreasing in beta, found in fp64 on [2^-8, 2^8] (an end of
// the interval when g has no sign change there; beta = 1 when no block
// reached k or all its logits are 0) by a safeguarded Newton iteration: each
// evaluation also sums g'(beta) = sum z^2 s (1 - s), a Newton step that
// leaves the current sign-change bracket is replaced by the bracket's
// geometric midpoint, and
// the iteration stops once a Newton step is below 2^-40 of beta (that step
// is taken; the next would be below the rounding noise of the sums, and tau
// is returned in fp32), or when the bracket is that narrow.  The
// convergence test comes before the bracket test: a converged step lands on
// the bracket end just moved and would otherwise fall back to bisection.  Each
// evaluation is one block-wide fp64 sum; every thread reads the same
// wavefront totals in the same order, so every decision is uniform.  Up to
// 8192 blocks the thread's values stay in registers, up to 24576 in LDS,
// beyond that they are re-read each evaluation with eight loads in flight
// per thread (from L2 after the first).
//
// Apply: c[r, k] = sigmoid(z[r, k] / tau[k]) in fp64, rounded once to fp32.
// Logits are clamped to [-64, 64], NaN -> 0, on both paths.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kFitThreads = 1024;
constexpr int kFitRegs = 8;      // blocks per thread held in registers
constexpr int kFitLds = 24576;   // blocks staged in LDS (5 bytes each)
constexpr int kFitBatch = 8;     // loads in flight per thread when streaming
constexpr double kBetaMin = 0.00390625, kBetaMax = 256.0;
constexpr int kMaxIter = 200;

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

// adds block i's terms of g and g' at beta
__device__ __forceinline__ void score_terms(double beta, float z, int code, double& g, double& gp) {
  const double zd = static_cast<double>(z);
  const double y = (code == 2) ? 1.0 : 0.0;
  const double sg = sigmoid64(beta * zd);
  g += (code == 0) ? 0.0 : zd * (sg - y);
  gp += (code == 0) ? 0.0 : zd * zd * sg * (1.0 - sg);
}

__device__ __forceinline__ double wave_sum64(double x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// MODE 0: values in registers (N <= kFitRegs * 1024); MODE 1: staged in LDS
// once (N <= kFitLds); MODE 2: re-read each evaluation, kFitBatch loads in
// flight per thread.
template <int MODE>
__global__ void __launch_bounds__(kFitThreads) sts_fit_kernel(dspark_sts_fit_args a) {
  // two slots per wavefront, alternating between evaluations, so one barrier
  // per evaluation suffices
  __shared__ double part[2][16][2];
  __shared__ int s_nz[16];
  __shared__ float zl[MODE == 1 ? kFitLds : 1];
  __shared__ unsigned char cl[MODE == 1 ? kFitLds : 1];
  const int k = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;

  float zr[MODE == 0 ? kFitRegs : 1];
  int cr[MODE == 0 ? kFitRegs : 1];
  int nonzero = 0;
  if (MODE == 0) {
#pragma unroll
    for (int j = 0; j < kFitRegs; ++j) {
      const int i = tid + j * kFitThreads;
      zr[j] = 0.0f;
      cr[j] = 0;
      if (i < N) fit_item(a, i, k, zr[j], cr[j]);
      nonzero |= (cr[j] != 0) & (zr[j] != 0.0f);
    }
  } else {
    for (int i0 = 0; i0 < N; i0 += kFitBatch * kFitThreads) {
      float zb[kFitBatch];
      int cb[kFitBatch];
#pragma unroll
      for (int j = 0; j < kFitBatch; ++j) {
        const int i = i0 + tid + j * kFitThreads;
        zb[j] = 0.0f;
        cb[j] = 0;
        if (i < N) fit_item(a, i, k, zb[j], cb[j]);
      }
#pragma unroll
      for (int j = 0; j < kFitBatch; ++j) {
        const int i = i0 + tid + j * kFitThreads;
        nonzero |= (cb[j] != 0) & (zb[j] != 0.0f);
        if (MODE == 1 && i < N) {
          zl[i] = zb[j];
          cl[i] = static_cast<unsigned char>(cb[j]);
        }
      }
    }
  }
  // block-wide "some reached logit is nonzero" (the barrier also publishes
  // the LDS copy)
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) nonzero |= __shfl_xor(nonzero, d);
  if (lane == 0) s_nz[wave] = nonzero;
  __syncthreads();
  int any_info = 0;
  for (int w = 0; w < 16; ++w) any_info |= s_nz[w];

  // g(beta) and g'(beta), block-wide; slot alternates between calls
  int slot = 0;
  auto score = [&](double beta, double& gp) -> double {
    double t = 0.0, tp = 0.0;
    if (MODE == 0) {
#pragma unroll
      for (int j = 0; j < kFitRegs; ++j) score_terms(beta, zr[j], cr[j], t, tp);
    } else if (MODE == 1) {
      for (int i = tid; i < N; i += kFitThreads) score_terms(beta, zl[i], cl[i], t, tp);
    } else {
      for (int i0 = 0; i0 < N; i0 += kFitBatch * kFitThreads) {
        float zb[kFitBatch];
        int cb[kFitBatch];
#pragma unroll
        for (int j = 0; j < kFitBatch; ++j) {
          const int i = i0 + tid + j * kFitThreads;
          zb[j] = 0.0f;
          cb[j] = 0;
          if (i < N) fit_item(a, i, k, zb[j], cb[j]);
        }
#pragma unroll
        for (int j = 0; j < kFitBatch; ++j) score_terms(beta, zb[j], cb[j], t, tp);
      }
    }
    t = wave_sum64(t);
    tp = wave_sum64(tp);
    if (lane == 0) {
      part[slot][wave][0] = t;
      part[slot][wave][1] = tp;
    }
    __syncthreads();
    double g = 0.0;
    gp = 0.0;
    for (int w = 0; w < 16; ++w) {
      g += part[slot][w][0];
      gp += part[slot][w][1];
    }
    slot ^= 1;
    return g;
  };

  double beta = 1.0;
  if (any_info) {
    double gp;
    const double g_lo = score(kBetaMin, gp);
    const double g_hi = score(kBetaMax, gp);
    if (g_lo >= 0.0) {
      beta = kBetaMin;
    } else if (g_hi <= 0.0) {
      beta = kBetaMax;
    } else {
      double lo = kBetaMin, hi = kBetaMax;  // g(lo) < 0 < g(hi)
      for (int it = 0; it < kMaxIter; ++it) {
        const double g = score(beta, gp);
        if (g == 0.0) break;
        if (g > 0.0) hi = beta;
        else lo = beta;
        const double step = g / gp;
        if (fabs(step) <= 0x1p-40 * beta) {  // converged (false for gp = 0 or NaN)
          beta -= step;
          break;
        }
        double next = beta - step;
        if (!(next > lo && next < hi)) next = sqrt(lo * hi);
        beta = next;
        if (hi - lo <= 0x1p-40 * beta) break;
      }
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
    hipLaunchKernelGGL(sts_fit_kernel<0>, dim3(a.gamma), dim3(kFitThreads), 0, s, a);
  else if (a.N <= kFitLds)
    hipLaunchKernelGGL(sts_fit_kernel<1>, dim3(a.gamma), dim3(kFitThreads), 0, s, a);
  else
    hipLaunchKernelGGL(sts_fit_kernel<2>, dim3(a.gamma), dim3(kFitThreads), 0, s, a);
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
