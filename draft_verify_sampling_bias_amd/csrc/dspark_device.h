// Device helpers shared by the libdspark kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dspark.h"

namespace dspark {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kIntMax = 0x7fffffff;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// bf16 bits of a finite float, rounded to nearest even.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// The RNN head's activation, and a state rounded to the nearest double-bf16
// value (hi = bf16(h), lo = bf16(h - hi), h = hi + lo: 16 significant bits),
// the form in which every consumer of the state reads it.
__device__ __forceinline__ float rnn_act(float z, int act) { return act == DSPARK_ACT_TANH ? tanhf(z) : z; }
__device__ __forceinline__ float double_bf16(float h) {
  const float hi = __uint_as_float(bf16_rne_bits(h) << 16);
  const float lo = __uint_as_float(bf16_rne_bits(h - hi) << 16);
  return hi + lo;
}

// 2^x on the hardware transcendental unit (v_exp_f32, 1 ulp).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// (m2, i2) beats (m, i): larger value, or equal value and lower index
// (evaluated without short-circuit branches)
__device__ __forceinline__ bool amax_takes(float m2, int i2, float m, int i) {
  return (static_cast<int>(m2 > m) | (static_cast<int>(m2 == m) & static_cast<int>(i2 < i))) != 0;
}

// Lane pairs (l, l ^ 16) and (l, l ^ 32) via the gfx950 permlane swaps (VALU,
// no LDS round trip): both lanes of a pair receive (x[lower lane], x[upper
// lane]) in that order, so a combine of the two is bit-identical in both.
__device__ __forceinline__ void lane_pair16(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  lo = r[0];
  hi = r[1];
}
__device__ __forceinline__ void lane_pair32(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  lo = r[0];
  hi = r[1];
}
// sum / (max, lowest index) over the lane pair l, l ^ 32
__device__ __forceinline__ float half_sum(float x) {
  uint32_t lo, hi;
  lane_pair32(__float_as_uint(x), lo, hi);
  return __uint_as_float(lo) + __uint_as_float(hi);
}
__device__ __forceinline__ void half_amax(float& m, int& i) {
  uint32_t ml, mh, il, ih;
  lane_pair32(__float_as_uint(m), ml, mh);
  lane_pair32(static_cast<uint32_t>(i), il, ih);
  const bool take =
      amax_takes(__uint_as_float(mh), static_cast<int>(ih), __uint_as_float(ml), static_cast<int>(il));
  m = __uint_as_float(take ? mh : ml);
  i = static_cast<int>(take ? ih : il);
}
// sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float quad_sum(float x) {
  uint32_t lo, hi;
  lane_pair16(__float_as_uint(x), lo, hi);
  x = __uint_as_float(lo) + __uint_as_float(hi);
  lane_pair32(__float_as_uint(x), lo, hi);
  return __uint_as_float(lo) + __uint_as_float(hi);
}
// maximum over the same four lanes
__device__ __forceinline__ float quad_max(float x) {
  uint32_t lo, hi;
  lane_pair16(__float_as_uint(x), lo, hi);
  x = fmaxf(__uint_as_float(lo), __uint_as_float(hi));
  lane_pair32(__float_as_uint(x), lo, hi);
  return fmaxf(__uint_as_float(lo), __uint_as_float(hi));
}
// (max, lowest index of the max) over the same four lanes
__device__ __forceinline__ void quad_amax(float& m, int& i) {
  uint32_t ml, mh, il, ih;
  lane_pair16(__float_as_uint(m), ml, mh);
  lane_pair16(static_cast<uint32_t>(i), il, ih);
  bool take = amax_takes(__uint_as_float(mh), static_cast<int>(ih), __uint_as_float(ml), static_cast<int>(il));
  m = __uint_as_float(take ? mh : ml);
  i = static_cast<int>(take ? ih : il);
  lane_pair32(__float_as_uint(m), ml, mh);
  lane_pair32(static_cast<uint32_t>(i), il, ih);
  take = amax_takes(__uint_as_float(mh), static_cast<int>(ih), __uint_as_float(ml), static_cast<int>(il));
  m = __uint_as_float(take ? mh : ml);
  i = static_cast<int>(take ? ih : il);
}

// 2^((x - m) c) for x <= m, with x == m giving 1 also when both are -inf (a
// vocabulary masked with -inf logits): the weight of a masked entry relative
// to a masked maximum stays finite, and relative to any finite maximum it is 0.
__device__ __forceinline__ float exp2_rel(float x, float m, float c) {
  return (x == m) ? 1.0f : __builtin_amdgcn_exp2f((x - m) * c);
}

// Scale that turns (logit - max) into a base-2 exponent at temperature T;
// 0 marks a greedy request (T <= 0 or NaN).  A positive T is used clamped
// to [1e-30, 1e30], so the scale stays finite and positive for a subnormal
// T and for T = +inf (at either end the fp32 softmax is already one-hot or
// uniform).
constexpr float kTempMin = 1e-30f, kTempMax = 1e30f;
__device__ __forceinline__ float temp_scale(float T) {
  return (T > 0.0f) ? (kLog2e / fminf(fmaxf(T, kTempMin), kTempMax)) : 0.0f;
}

// (m, i) <- better of (m, i) and (m2, i2): larger value, lower index on ties.
__device__ __forceinline__ void amax_merge(float& m, int& i, float m2, int i2) {
  const bool take = (static_cast<int>(m2 > m) | (static_cast<int>(m2 == m) & static_cast<int>(i2 < i))) != 0;
  m = take ? m2 : m;
  i = take ? i2 : i;
}

__device__ __forceinline__ void wave_amax(float& m, int& i) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    float m2 = __shfl_xor(m, d);
    int i2 = __shfl_xor(i, d);
    amax_merge(m, i, m2, i2);
  }
}

// Butterfly sum: every lane ends with the same bits (a + b == b + a).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

__device__ __forceinline__ int wave_min_int(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = min(x, __shfl_xor(x, d));
  return x;
}

__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, __shfl_xor(x, d));
  return x;
}

// v of the lane that DPP control CTRL names, 0 where it names none or the
// row is outside ROW_MASK (VALU data-parallel primitives, no LDS round trip)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive scan inside a wavefront (fixed order): Hillis-Steele inside each
// 16-lane row (row_shr 1, 2, 4, 8), then row 0's total into row 1 and row
// 2's into row 3 (row_bcast:15), then row 1's running total into rows 2 and
// 3 (row_bcast:31).
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_or_zero<0x111, 0xf>(v);
  v += dpp_or_zero<0x112, 0xf>(v);
  v += dpp_or_zero<0x114, 0xf>(v);
  v += dpp_or_zero<0x118, 0xf>(v);
  v += dpp_or_zero<0x142, 0xa>(v);
  v += dpp_or_zero<0x143, 0xc>(v);
  return v;
}

// Block-wide (256 threads = 4 waves) inclusive scan.  Returns the inclusive
// prefix of this thread; *excl gets the exclusive prefix, computed so that
// the intervals [excl, incl) of consecutive threads meet exactly; *total is
// the sum over the block (equal to the last thread's inclusive prefix).
// `lds` needs 4 floats.  Contains two __syncthreads().
__device__ __forceinline__ float block256_scan(float x, float* lds, float* excl, float* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float v = wave_incl_scan(x);
  if (lane == 63) lds[wave] = v;
  __syncthreads();
  const float w0 = lds[0], w1 = lds[1], w2 = lds[2], w3 = lds[3];
  __syncthreads();
  float off = 0.0f;
  if (wave == 1) off = w0;
  if (wave == 2) off = w0 + w1;
  if (wave == 3) off = (w0 + w1) + w2;
  const float incl = off + v;
  const float prev = __shfl_up(incl, 1);
  *excl = (lane == 0) ? off : prev;
  *total = ((w0 + w1) + w2) + w3;
  return incl;
}

// Block-wide (256 threads) argmax with lowest-index ties; all threads get it.
// `lm`, `li` need 4 entries each.  Contains two __syncthreads().
__device__ __forceinline__ void block256_amax(float& m, int& i, float* lm, int* li) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_amax(m, i);
  if (lane == 0) {
    lm[wave] = m;
    li[wave] = i;
  }
  __syncthreads();
  m = lm[0];
  i = li[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) amax_merge(m, i, lm[w], li[w]);
  __syncthreads();
}

// Block-wide (256 threads) min / max of an int; all threads get it.
__device__ __forceinline__ int block256_min_int(int x, int* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_min_int(x);
  if (lane == 0) lds[wave] = x;
  __syncthreads();
  x = min(min(lds[0], lds[1]), min(lds[2], lds[3]));
  __syncthreads();
  return x;
}

__device__ __forceinline__ int block256_max_int(int x, int* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_max_int(x);
  if (lane == 0) lds[wave] = x;
  __syncthreads();
  x = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
  __syncthreads();
  return x;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace dspark
