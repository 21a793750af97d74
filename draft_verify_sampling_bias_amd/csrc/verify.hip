// Verify kernels ("DSpark" explainer sections 2-3; llama.cpp PR #25173,
// "Losslessness").
//
// verify_stats: one wavefront per (target row, 4096-entry chunk), the
//   request given by the grid; coalesced float4 sweep giving each (row,
//   chunk) its maximum, lowest argmax and, for a sampled request, sum of
//   exp((t - max)/T).  This is the pass that reads every target logit once.
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

// verify_stats: workgroup (r, j, g) covers chunks 4g .. 4g + 3 of row j of
// request r (row row_offsets[r] + j; workgroups past the request's last row
// leave at once), one chunk per wavefront: 16 float4 loads per lane (1 KB
// contiguous per instruction), then wavefront-level reductions only (no
// workgroup barrier).
template <bool VEC4>
__device__ __forceinline__ void chunk_load(const float* row, int base, int V, int lane, float (&x)[64]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int v = base + (j * 64 + lane) * 4;
    if (VEC4) {
      // read once: non-temporal, so the stream does not displace the Markov
      // weights that the residual pass reads next from the last-level cache
      const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(row + min(v, V - 4)));
      x[4 * j + 0] = t[0];
      x[4 * j + 1] = t[1];
      x[4 * j + 2] = t[2];
      x[4 * j + 3] = t[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = __builtin_nontemporal_load(row + min(v + e, V - 1));
    }
  }
}

template <bool VEC4>
__global__ void __launch_bounds__(256) verify_stats_kernel(VerifyParams p) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  // the residual list is rebuilt by verify_finish, which runs after this kernel
  if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) {
    if (p.rs_count != nullptr) *p.rs_count = 0;
    if (p.err_clear != nullptr) *p.err_clear = 0u;
  }
  const int ch = blockIdx.z * 4 + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (ch >= p.n_chunks) return;  // wavefront-uniform; no workgroup barrier follows
  const int64_t lo = min(max(static_cast<int64_t>(p.row_offsets[r]), int64_t{0}), p.n_rows);
  const int64_t hi = min(max(static_cast<int64_t>(p.row_offsets[r + 1]), lo), p.n_rows);
  const int64_t row = lo + blockIdx.y;
  if (row >= hi) return;
  const float c = temp_scale(p.temp[r]);
  const int V = p.V;
  const int base = ch * kChunk;
  float x[64];
  chunk_load<VEC4>(p.target + row * V, base, V, lane, x);
  float m = -INFINITY;
  int im = kIntMax;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = base + (j * 64 + lane) * 4 + e;
      // lowest index of the maximum, also when every entry is -inf
      const bool gt = (v < V) & amax_takes(x[4 * j + e], v, m, im);
      m = gt ? x[4 * j + e] : m;
      im = gt ? v : im;
    }
  wave_amax(m, im);
  float sum = 0.0f;
  if (c > 0.0f) {  // workgroup-uniform (one request per workgroup)
    float e_loc = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = base + (j * 64 + lane) * 4 + e;
        const float w = exp2_rel(x[4 * j + e], m, c);
        e_loc += (v < V) ? w : 0.0f;
      }
    sum = wave_sum(e_loc);
  }
  if (lane == 0) {
    float* rec = p.vpart + (row * p.n_chunks + ch) * kChunkFloats;
    *reinterpret_cast<f32x4_t*>(rec) = f32x4_t{m, __int_as_float(im), sum, 0.0f};
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
  const int64_t og = static_cast<int64_t>(n) * gamma;
  // every input that depends only on n is loaded first, in one batch; lane j
  // of each wavefront holds position j's draft values
  const int64_t i0 = p.row_offsets[n], i1 = p.row_offsets[n + 1];
  const float T = p.temp[n];
  const float uf = p.u_final[n];
  const int anc = p.anchor[n];
  int yv = 0;
  float qt = 1.0f, ua = 0.0f, qs0 = 0.0f, qs1 = 1.0f;
  if (lane < gamma) {
    const int64_t o = og + lane;
    yv = p.y[o];
    qt = p.q_tok[o];
    ua = p.u_accept[o];
    qs0 = p.q_stats[2 * o];
    qs1 = p.q_stats[2 * o + 1];
  }
  const int64_t nrows = i1 - i0;
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
  const float c = temp_scale(T);
  yv = clampi(yv, 0, V - 1);
  // target logit of each drafted token (rows i0 + j, j < l), in flight while
  // the chunk records below are combined
  float tl = 0.0f;
  if (wave == 0 && lane < l && c > 0.0f) tl = p.target[(i0 + lane) * V + yv];

  for (int j = wave; j <= l; j += 4) {
    const f32x4_t* rec = reinterpret_cast<const f32x4_t*>(p.vpart + (i0 + j) * p.n_chunks * kChunkFloats);
    float m = -INFINITY;
    int im = kIntMax;
    for (int ch = lane; ch < p.n_chunks; ch += 64) {
      const f32x4_t r = rec[ch];
      amax_merge(m, im, r[0], __float_as_int(r[1]));
    }
    wave_amax(m, im);
    float z = 0.0f;
    if (c > 0.0f) {
      for (int ch = lane; ch < p.n_chunks; ch += 64) {
        const f32x4_t r = rec[ch];
        z += r[2] * exp2_hw((r[0] - m) * c);
      }
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
      if (c == 0.0f) {
        const bool ok = (yv == rI[lane]);
        pt = ok ? 1.0f : 0.0f;
        rej = !ok;
      } else {
        pt = exp2_hw((tl - rM[lane]) * c) / rZ[lane];
        const float ratio = pt / qt;
        rej = !(ua < ratio);
      }
    }
    const unsigned long long mask = __ballot(rej);
    const int nacc = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : l;
    if (lane < gamma) p.p_tok[og + lane] = (lane < l) ? pt : 0.0f;
    // a sampled rejection: hand (prev, U row, target row, q and p statistics)
    // to the residual pass; every value is already in this wavefront
    const float q0 = __shfl(qs0, nacc & 63), q1 = __shfl(qs1, nacc & 63);
    const int yprev = __shfl(yv, (nacc - 1) & 63);
    if (lane == 0) {
      p.n_accept[n] = nacc;
      s_nacc = nacc;
      if (c != 0.0f && nacc < l) {
        const int prev = (nacc == 0) ? anc : yprev;
        int32_t* inf = p.rs_info + 4 * static_cast<int64_t>(n);
        inf[0] = 1;
        inf[1] = clampi(prev, 0, V - 1);
        inf[2] = static_cast<int32_t>(og + nacc);
        inf[3] = static_cast<int32_t>(i0 + nacc);
        float* st = p.rs_stats + 4 * static_cast<int64_t>(n);
        st[0] = q0;
        st[1] = q1;
        st[2] = rM[nacc];
        st[3] = rZ[nacc];
        if (p.rs_list != nullptr) {
          // slot order varies from run to run; each entry carries its request
          // and the residual pass writes that request's records only
          const int slot = atomicAdd(p.rs_count, 1);
          ResidualEntry e;
          e.n = n;
          e.prev = inf[1];
          e.urow = inf[2];
          e.trow = inf[3];
          e.Mq = q0;
          e.Zq = q1;
          e.Mp = rM[nacc];
          e.Zp = rZ[nacc];
          e.T = T;
          e.pad[0] = e.pad[1] = e.pad[2] = 0.0f;
          p.rs_list[slot] = e;
        }
      }
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
    const float u = clamp_uniform(uf);
    const int out = chunk_draw(p.vpart + (i0 + l) * p.n_chunks * kChunkFloats, p.n_chunks, p.target + (i0 + l) * V,
                               V, rM[l], c, u, &sh);
    if (tid == 0) {
      p.out_tok[n] = (out >= 0) ? out : rI[l];
      clear_residual(p, n);
    }
  }
}

}  // namespace

hipError_t launch_verify_stats(const VerifyParams& p, hipStream_t s) {
  if (p.R == 0 || p.n_rows == 0) return hipSuccess;
  // y: row index within the request (at most gamma + 1 rows)
  const dim3 grid(static_cast<unsigned>(p.R), static_cast<unsigned>(p.gamma + 1),
                  static_cast<unsigned>((p.n_chunks + 3) / 4));
  if ((p.V & 3) == 0)
    hipLaunchKernelGGL(verify_stats_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(verify_stats_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_verify_finish(const VerifyParams& p, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  hipLaunchKernelGGL(verify_finish_kernel, dim3(p.R), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
