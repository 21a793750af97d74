// Hardware-aware capacity ("DSpark" explainer sections 9 and 10): the number
// of draft positions K that the next verify batch should hold, chosen by the
// causal greedy on the expected effective output times the engine's step rate.
//
//   candidates  the survival values of an earlier step (clamped to [0, 1],
//               NaN -> 0), taken largest first;
//   E(K)        R + the sum of the K largest values, rounded once to fp64
//               from the exact sum, then added to R in fp64;
//   Theta(K)    E(K) * SPS[R + K] in fp64 (R anchor rows plus K draft rows);
//   K           the first K < kmax with Theta(K + 1) <= Theta(K) (or NaN),
//               else kmax = min(R * gamma, n_sps - 1 - R).
//
// One workgroup of 1024 threads, each holding E = 2, 4, 8 or 16 entries
// (N = 1024 E >= R * gamma, padded with +0):
//   1. the values' fp32 bit patterns (non-negative, so their unsigned order
//      is the value order) are sorted descending by a bitonic network: strides
//      below E inside a thread's registers, below 64 E by lane shuffles, the
//      ten cross-wavefront stages through LDS;
//   2. thread t then owns sorted positions t*E .. t*E + E - 1 and sums them
//      exactly in a 192-bit fixed-point integer (unit 2^-149, the smallest
//      fp32 subnormal; a value <= 1 is below 2^150 and at most 2^14 of them
//      are summed); a block-wide exclusive scan of those integers gives every
//      exact prefix sum;
//   3. each prefix sum is rounded to fp64 (round to nearest even), R is added
//      and the stop test is evaluated for each owned position; a block
//      minimum gives K.
// The arithmetic after the exact sum (one rounding to fp64, one fp64 add, one
// fp64 multiply, a strict comparison) is the definition's, so K, E(K) and
// Theta(K) do not depend on the summation order.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kCapThreads = 1024;

struct U192 {
  unsigned long long w0, w1, w2;
};

__host__ __device__ __forceinline__ U192 u192_add(const U192& a, const U192& b) {
  U192 r;
  r.w0 = a.w0 + b.w0;
  const unsigned long long c0 = r.w0 < a.w0 ? 1ull : 0ull;
  const unsigned long long t1 = a.w1 + b.w1;
  const unsigned long long c1a = t1 < a.w1 ? 1ull : 0ull;
  r.w1 = t1 + c0;
  const unsigned long long c1b = r.w1 < t1 ? 1ull : 0ull;
  r.w2 = a.w2 + b.w2 + c1a + c1b;
  return r;
}

// An fp32 value in [0, 1] (bit pattern, sign clear) as an integer multiple
// of 2^-149: subnormal m -> m; normal (e, m) -> (2^23 + m) << (e - 1).
__host__ __device__ __forceinline__ U192 u192_from_f32_bits(unsigned int b) {
  const unsigned int e = (b >> 23) & 0xffu;
  const unsigned long long m = b & 0x7fffffu;
  const unsigned long long mant = e ? (m | 0x800000ull) : m;
  const int s = e ? static_cast<int>(e) - 1 : 0;  // 0 .. 126
  const int off = s & 63;
  const unsigned long long lo = mant << off;
  const unsigned long long hi = off ? (mant >> (64 - off)) : 0ull;
  U192 r;
  r.w0 = (s < 64) ? lo : 0ull;
  r.w1 = (s < 64) ? hi : lo;
  r.w2 = (s < 64) ? 0ull : hi;
  return r;
}

// 64 bits of x starting at bit pos (0 <= pos < 192); bits past 191 read 0.
__host__ __device__ __forceinline__ unsigned long long u192_bits_at(const U192& x, int pos) {
  const int limb = pos >> 6, off = pos & 63;
  const unsigned long long lo = limb == 0 ? x.w0 : (limb == 1 ? x.w1 : x.w2);
  const unsigned long long hi = limb == 0 ? x.w1 : (limb == 1 ? x.w2 : 0ull);
  return off ? ((lo >> off) | (hi << (64 - off))) : lo;
}

// whether any bit below position pos (0 <= pos <= 192) is set
__host__ __device__ __forceinline__ bool u192_any_below(const U192& x, int pos) {
  auto part = [](unsigned long long w, int nbits) -> bool {
    if (nbits <= 0) return false;
    if (nbits >= 64) return w != 0ull;
    return (w & ((1ull << nbits) - 1ull)) != 0ull;
  };
  return part(x.w0, pos) || part(x.w1, pos - 64) || part(x.w2, pos - 128);
}

// x * 2^-149 rounded to the nearest fp64 (ties to even).
__host__ __device__ __forceinline__ double u192_to_double(const U192& x) {
  int h;
  if (x.w2) h = 128 + 63 - __builtin_clzll(x.w2);
  else if (x.w1) h = 64 + 63 - __builtin_clzll(x.w1);
  else if (x.w0) h = 63 - __builtin_clzll(x.w0);
  else return 0.0;
  if (h <= 52) return ldexp(static_cast<double>(x.w0), -149);  // exact
  int sh = h - 52;  // the 53-bit significand is bits sh .. h
  unsigned long long mant = u192_bits_at(x, sh) & ((1ull << 53) - 1ull);
  const bool round_bit = (u192_bits_at(x, sh - 1) & 1ull) != 0ull;
  const bool sticky = u192_any_below(x, sh - 1);
  if (round_bit && (sticky || (mant & 1ull))) {
    ++mant;
    if (mant == (1ull << 53)) {
      mant >>= 1;
      ++sh;
    }
  }
  return ldexp(static_cast<double>(mant), sh - 149);
}

__device__ __forceinline__ U192 u192_shfl_up(const U192& x, int d) {
  U192 r;
  r.w0 = __shfl_up(x.w0, d);
  r.w1 = __shfl_up(x.w1, d);
  r.w2 = __shfl_up(x.w2, d);
  return r;
}

// Compare-exchange of element g with its bitonic partner value pv at
// stride j of merge size k: keeps the larger value where g is the first of
// its pair in a descending block or the second in an ascending one.
__device__ __forceinline__ unsigned int bitonic_keep(unsigned int v, unsigned int pv, int g, int j, int k) {
  const bool take_max = ((g & j) == 0) == ((g & k) == 0);
  return take_max ? max(v, pv) : min(v, pv);
}

// E = sorted values per thread (2, 4, 8 or 16): N = 1024 * E entries.
template <int E>
__global__ void __launch_bounds__(kCapThreads) capacity_kernel(dspark_capacity_args a) {
  constexpr int N = kCapThreads * E;
  // exchange buffer of the cross-wavefront stages ([e][thread], so that a
  // wavefront's lanes touch consecutive words), then the rates SPS[R + i]
  __shared__ unsigned int xbuf[DSPARK_CAPACITY_MAX_CANDIDATES + 1];
  __shared__ unsigned long long wtot[16 * 3];  // wavefront totals of the scan
  __shared__ int s_kmin[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.R;
  const int n = R * a.gamma;
  const int kmax = min(n, a.n_sps - 1 - R);
  const int base = tid * E;  // this thread holds entries base .. base + E - 1

  // load, clamp (NaN -> 0, -0 -> +0) and pad with +0
  unsigned int v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float x = 0.0f;
    if (base + e < n) {
      x = fminf(fmaxf(a.a_lag[base + e], 0.0f), 1.0f);
      if (x == 0.0f) x = 0.0f;
    }
    v[e] = __float_as_uint(x);
  }

  // bitonic sort, descending: strides below E inside the thread, below 64 E
  // across the lanes of a wavefront, the rest through LDS
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64 * E) {
        const int m = j / E;  // partner thread tid ^ m, another wavefront
#pragma unroll
        for (int e = 0; e < E; ++e) xbuf[e * kCapThreads + tid] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = bitonic_keep(v[e], xbuf[e * kCapThreads + (tid ^ m)], base + e, j, k);
        __syncthreads();
      } else if (j >= E) {
        const int m = j / E;  // partner lane lane ^ m
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = bitonic_keep(v[e], __shfl_xor(v[e], m), base + e, j, k);
      } else {
#pragma unroll
        for (int jj = E / 2; jj >= 1; jj >>= 1) {
          if (jj == j) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              if ((e & jj) == 0) {
                const unsigned int x = v[e], y = v[e | jj];
                const bool desc = ((base + e) & k) == 0;
                v[e] = desc ? max(x, y) : min(x, y);
                v[e | jj] = desc ? min(x, y) : max(x, y);
              }
            }
          }
        }
      }
    }
  }

  // the rates the stop tests read, SPS[R + i] for i = 0 .. kmax, into LDS
  float* sps_s = reinterpret_cast<float*>(xbuf);
  for (int i = tid; i <= kmax; i += kCapThreads) sps_s[i] = a.sps[R + i];

  // block-wide exclusive scan of the exact partial sums
  U192 local = {0ull, 0ull, 0ull};
#pragma unroll
  for (int e = 0; e < E; ++e) local = u192_add(local, u192_from_f32_bits(v[e]));
  U192 incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const U192 o = u192_shfl_up(incl, d);
    if (lane >= d) incl = u192_add(incl, o);
  }
  if (lane == 63) {
    wtot[3 * wave] = incl.w0;
    wtot[3 * wave + 1] = incl.w1;
    wtot[3 * wave + 2] = incl.w2;
  }
  __syncthreads();  // also orders the rate stores before the reads below
  U192 excl = {0ull, 0ull, 0ull};
  for (int w = 0; w < wave; ++w) {
    const U192 t = {wtot[3 * w], wtot[3 * w + 1], wtot[3 * w + 2]};
    excl = u192_add(excl, t);
  }
  const U192 o = u192_shfl_up(incl, 1);
  if (lane > 0) excl = u192_add(excl, o);

  // stop tests for the owned positions i = base + e < kmax
  const double Rd = static_cast<double>(R);
  U192 S = excl;
  double E_now = __dadd_rn(Rd, u192_to_double(S));
  int kfirst = kmax;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = base + e;
    if (i < kmax) {
      S = u192_add(S, u192_from_f32_bits(v[e]));
      const double E_next = __dadd_rn(Rd, u192_to_double(S));
      const double th_now = __dmul_rn(E_now, static_cast<double>(sps_s[i]));
      const double th_next = __dmul_rn(E_next, static_cast<double>(sps_s[i + 1]));
      if (!(th_next > th_now) && i < kfirst) kfirst = i;
      E_now = E_next;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) kfirst = min(kfirst, __shfl_xor(kfirst, d));
  if (lane == 0) s_kmin[wave] = kfirst;
  __syncthreads();
  int K = s_kmin[0];
  for (int w = 1; w < 16; ++w) K = min(K, s_kmin[w]);

  // the thread owning position K (the last thread for K = N) writes E(K)
  // and Theta(K)
  const int owner = min(K / E, kCapThreads - 1);
  if (tid == owner) {
    U192 SK = excl;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (base + e < K) SK = u192_add(SK, u192_from_f32_bits(v[e]));
    const double Ek = __dadd_rn(Rd, u192_to_double(SK));
    a.K[0] = K;
    if (a.expected) a.expected[0] = Ek;
    if (a.theta) a.theta[0] = __dmul_rn(Ek, static_cast<double>(sps_s[K]));
  }
}

}  // namespace

hipError_t launch_capacity(const dspark_capacity_args& a, hipStream_t s) {
  const int n = a.R * a.gamma;
  if (n <= 2 * kCapThreads)
    hipLaunchKernelGGL(capacity_kernel<2>, dim3(1), dim3(kCapThreads), 0, s, a);
  else if (n <= 4 * kCapThreads)
    hipLaunchKernelGGL(capacity_kernel<4>, dim3(1), dim3(kCapThreads), 0, s, a);
  else if (n <= 8 * kCapThreads)
    hipLaunchKernelGGL(capacity_kernel<8>, dim3(1), dim3(kCapThreads), 0, s, a);
  else
    hipLaunchKernelGGL(capacity_kernel<16>, dim3(1), dim3(kCapThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
