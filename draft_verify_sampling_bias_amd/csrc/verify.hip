// Verify kernels ("DSpark" explainer sections 2-3; llama.cpp PR #25173,
// "Losslessness").
//
// verify_stats: one workgroup per (target row, 4096-entry chunk); coalesced
//   float4 sweep of the row giving the chunk's maximum, lowest argmax and, for
//   a sampled request, sum of exp((t - max)/T).  This is the pass that reads
//   every target logit once.
// verify_finish: one workgroup per request; combines its rows' chunk records
//   into (max, argmax, Z) per row, runs the accept tests u < p/q left to
//   right, finds the first rejection, and emits the greedy correction/bonus
//   or the sampled bonus (inverse CDF over the bonus row).  A sampled
//   rejection is handed to the residual pass (bias_tile.hip residual mode,
//   finish.hip residual_finish_kernel).

#include "dspark_device.h"
#include "launchers.h"
#include "plan.h"
#include "sample_device.h"

namespace dspark {
namespace {

constexpr int kOffLds = 4096;  // row_offsets entries staged in LDS

// first index i in [0, n) with off[i] > key, or n
__device__ __forceinline__ int upper_bound_i32(const int32_t* off, int n, int64_t key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(off[mid]) > key)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

__global__ void __launch_bounds__(256) verify_stats_kernel(VerifyParams p) {
  __shared__ int32_t s_off[kOffLds];
  __shared__ float fred[4];
  __shared__ int ired[4];
  __shared__ int s_req;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t row = b / p.n_chunks;
  const int ch = static_cast<int>(b - row * p.n_chunks);
  const int V = p.V;
  const float* tr = p.target + row * V;
  const int base = ch * kChunk;
  const bool vec4 = (V & 3) == 0;

  float x[16];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int v = base + (it * 256 + tid) * 4;
    if (vec4 && v < V) {
      const f32x4_t t = *reinterpret_cast<const f32x4_t*>(tr + v);
      x[4 * it + 0] = t[0];
      x[4 * it + 1] = t[1];
      x[4 * it + 2] = t[2];
      x[4 * it + 3] = t[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * it + e] = (v + e < V) ? tr[v + e] : -INFINITY;
    }
  }

  // request owning this row
  int r;
  if (p.R + 1 <= kOffLds) {
    for (int i = tid; i <= p.R; i += 256) s_off[i] = p.row_offsets[i];
    __syncthreads();
    r = upper_bound_i32(s_off, p.R + 1, row) - 1;
  } else {
    if (tid == 0) s_req = upper_bound_i32(p.row_offsets, p.R + 1, row) - 1;
    __syncthreads();
    r = s_req;
  }
  r = clampi(r, 0, p.R - 1);
  const float c = temp_scale(p.temp[r]);

  float m = -INFINITY;
  int im = kIntMax;
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = base + (it * 256 + tid) * 4 + e;
      if (v < V && x[4 * it + e] > m) {
        m = x[4 * it + e];
        im = v;
      }
    }
  block256_amax(m, im, fred, ired);

  float sum = 0.0f;
  if (c > 0.0f) {
    float e_loc = 0.0f;
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = base + (it * 256 + tid) * 4 + e;
        if (v < V) e_loc += exp2_rel(x[4 * it + e], m, c);
      }
    e_loc = wave_sum(e_loc);
    if ((tid & 63) == 0) fred[tid >> 6] = e_loc;
    __syncthreads();
    sum = ((fred[0] + fred[1]) + fred[2]) + fred[3];
  }
  if (tid == 0) {
    float* rec = p.vpart + (row * p.n_chunks + ch) * kChunkFloats;
    rec[0] = m;
    rec[1] = __int_as_float(im);
    rec[2] = sum;
    rec[3] = 0.0f;
  }
}

// marks request n as needing no residual pass (all four words written)
__device__ __forceinline__ void clear_residual(const VerifyParams& p, int n) {
  int32_t* inf = p.rs_info + 4 * static_cast<int64_t>(n);
  inf[0] = 0;
  inf[1] = 0;
  inf[2] = 0;
  inf[3] = 0;
}

__global__ void __launch_bounds__(256) verify_finish_kernel(VerifyParams p) {
  __shared__ float rM[DSPARK_MAX_GAMMA + 1], rZ[DSPARK_MAX_GAMMA + 1];
  __shared__ int rI[DSPARK_MAX_GAMMA + 1];
  __shared__ int s_nacc;
  __shared__ ChunkScratch sh;
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = p.V, gamma = p.gamma;
  const int64_t i0 = p.row_offsets[n], i1 = p.row_offsets[n + 1];
  const int64_t nrows = i1 - i0;
  const int64_t og = static_cast<int64_t>(n) * gamma;
  if (nrows < 1 || nrows > gamma + 1 || i0 < 0 || i1 > p.n_rows) {
    // inconsistent offsets: defined, in-bounds outputs
    if (tid < gamma) p.p_tok[og + tid] = 0.0f;
    if (tid == 0) {
      p.n_accept[n] = 0;
      p.out_tok[n] = -1;
      clear_residual(p, n);
    }
    return;
  }
  const int l = static_cast<int>(nrows) - 1;
  const float c = temp_scale(p.temp[n]);

  for (int j = wave; j <= l; j += 4) {
    const float* rec = p.vpart + (i0 + j) * p.n_chunks * kChunkFloats;
    float m = -INFINITY;
    int im = kIntMax;
    for (int ch = lane; ch < p.n_chunks; ch += 64)
      amax_merge(m, im, rec[ch * kChunkFloats], __float_as_int(rec[ch * kChunkFloats + 1]));
    wave_amax(m, im);
    float z = 0.0f;
    if (c > 0.0f) {
      for (int ch = lane; ch < p.n_chunks; ch += 64)
        z += rec[ch * kChunkFloats + 2] * exp2_hw((rec[ch * kChunkFloats] - m) * c);
      z = wave_sum(z);
    }
    if (lane == 0) {
      rM[j] = m;
      rI[j] = clampi(im, 0, V - 1);
      rZ[j] = z;
    }
  }
  __syncthreads();

  if (wave == 0) {
    bool rej = false;
    float pt = 0.0f;
    if (lane < l) {
      const int64_t o = og + lane;
      const int yj = clampi(p.y[o], 0, V - 1);
      if (c == 0.0f) {
        const bool ok = (yj == rI[lane]);
        pt = ok ? 1.0f : 0.0f;
        rej = !ok;
      } else {
        const float t = p.target[(i0 + lane) * V + yj];
        pt = exp2_hw((t - rM[lane]) * c) / rZ[lane];
        const float ratio = pt / p.q_tok[o];
        rej = !(p.u_accept[o] < ratio);
      }
    }
    const unsigned long long mask = __ballot(rej);
    const int nacc = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : l;
    if (lane < gamma) p.p_tok[og + lane] = (lane < l) ? pt : 0.0f;
    if (lane == 0) {
      p.n_accept[n] = nacc;
      s_nacc = nacc;
    }
  }
  __syncthreads();
  const int nacc = s_nacc;

  if (c == 0.0f) {
    if (tid == 0) {
      p.out_tok[n] = rI[nacc];
      clear_residual(p, n);
    }
    return;
  }
  if (nacc == l) {
    const float u = clamp_uniform(p.u_final[n]);
    const int out = chunk_draw(p.vpart + (i0 + l) * p.n_chunks * kChunkFloats, p.n_chunks, p.target + (i0 + l) * V,
                               V, rM[l], c, u, &sh);
    if (tid == 0) {
      p.out_tok[n] = (out >= 0) ? out : rI[l];
      clear_residual(p, n);
    }
  } else if (tid == 0) {
    const int prev = (nacc == 0) ? p.anchor[n] : p.y[og + nacc - 1];
    int32_t* inf = p.rs_info + 4 * static_cast<int64_t>(n);
    inf[0] = 1;
    inf[1] = clampi(prev, 0, V - 1);
    inf[2] = static_cast<int32_t>(og + nacc);
    inf[3] = static_cast<int32_t>(i0 + nacc);
    const float* qs = p.q_stats + 2 * (og + nacc);
    float* st = p.rs_stats + 4 * static_cast<int64_t>(n);
    st[0] = qs[0];
    st[1] = qs[1];
    st[2] = rM[nacc];
    st[3] = rZ[nacc];
  }
}

}  // namespace

hipError_t launch_verify_stats(const VerifyParams& p, hipStream_t s) {
  if (p.R == 0 || p.n_rows == 0) return hipSuccess;
  const int64_t blocks = p.n_rows * p.n_chunks;
  hipLaunchKernelGGL(verify_stats_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_verify_finish(const VerifyParams& p, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  hipLaunchKernelGGL(verify_finish_kernel, dim3(p.R), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
