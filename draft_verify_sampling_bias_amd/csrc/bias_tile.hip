// Fused Markov bias + softmax statistics over the vocabulary (gfx950).
//
// The Markov head's bias for request n is B[n, v] = sum_j W2[v, j] * W1[prev_n, j]
// ("DSpark" explainer, section 7; llama.cpp PR #25173 description:
// bias(prev) = markov_w2 . markov_w1[prev]).  For a batch of requests this is
// the product B^T = W2 . H^T with H = W1[prev] gathered row by row.  One
// workgroup owns 128 vocabulary rows (four wavefronts of 32) and all requests:
// each W2 row is read from HBM once per position and stays in registers as
// MFMA A fragments while every request chunk streams past it, so the work is
// bound by the W2 + U streams, with the contraction on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  The epilogue adds the base
// logits U and reduces each request's 128 values in registers and LDS to a
// small record; neither B nor s = U + B is ever written to memory.
//
// MFMA operand layout (32x32 output, wave64): A lane l holds row (l & 31),
// 8 consecutive k at 8 * (l >> 5); B lane l holds column (l & 31), the same k;
// accumulator element i of lane l is row 8*(i/4) + 4*(l>>5) + (i%4), column
// (l & 31).  Here rows are vocabulary entries and columns are requests.

#include "dspark_device.h"
#include "launchers.h"
#include "plan.h"

namespace dspark {
namespace {

constexpr int kNchBf16 = 64;  // requests per chunk: two 32-wide MFMA column blocks
constexpr int kNchF32 = 32;   // requests per chunk in the fp32-weight kernel

// Loads this lane's 16 logits of one request row: rows vw + 8g + 4*khalf + e,
// g = 0..3, e = 0..3.  Entries past V, or of an inactive request, read as -inf.
__device__ __forceinline__ void load_row16(const float* __restrict__ row, int vbase, int V, bool vec4,
                                           bool ok, float (&x)[16]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int v = vbase + 8 * g;
    if (ok && vec4 && v < V) {
      const f32x4_t t = *reinterpret_cast<const f32x4_t*>(row + v);
      x[4 * g + 0] = t[0];
      x[4 * g + 1] = t[1];
      x[4 * g + 2] = t[2];
      x[4 * g + 3] = t[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * g + e] = (ok && v + e < V) ? row[v + e] : -INFINITY;
    }
  }
}

__device__ __forceinline__ int acc_row(int i, int khalf) { return 8 * (i >> 2) + 4 * khalf + (i & 3); }

// Per-request values staged in LDS for one chunk.
struct ChunkInfo {
  int act, prev, urow, trow;
  float c, Mq, iZq, Mp, iZp;
};

__device__ __forceinline__ ChunkInfo fetch_info(const TileParams& p, int n, bool resid) {
  ChunkInfo ci{0, 0, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n >= p.R) return ci;
  ci.c = temp_scale(p.temp[n]);
  if (!resid) {
    ci.act = 1;
    ci.prev = p.prev_base[static_cast<int64_t>(n) * p.prev_stride];
  } else {
    const int32_t* inf = p.rs_info + 4 * static_cast<int64_t>(n);
    ci.act = inf[0];
    ci.prev = inf[1];
    ci.urow = inf[2];
    ci.trow = inf[3];
    const float* st = p.rs_stats + 4 * static_cast<int64_t>(n);
    ci.Mq = st[0];
    ci.iZq = 1.0f / st[1];
    ci.Mp = st[2];
    ci.iZp = 1.0f / st[3];
  }
  ci.prev = clampi(ci.prev, 0, p.V - 1);
  return ci;
}

// Draft epilogue, phase 1: s = acc + U (in place in x), per-lane then per-wave
// max / lowest argmax of this wave's 32 rows for the lane's request.
__device__ __forceinline__ void draft_phase1(const f32x16_t& acc, float (&x)[16], int vw, int khalf,
                                             int V, float* wm, int* wi) {
  float m = -INFINITY;
  int im = kIntMax;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = vw + acc_row(i, khalf);
    const float s = acc[i] + x[i];
    x[i] = s;
    if (v < V && s > m) {
      m = s;
      im = v;
    }
  }
  amax_merge(m, im, __shfl_xor(m, 32), __shfl_xor(im, 32));
  if (khalf == 0) {
    *wm = m;
    *wi = im;
  }
}

// Draft epilogue, phase 2: tile max from the four wave maxima, then this
// wave's sum of exp((s - M)/T); lane (khalf == 0) writes the record.
__device__ __forceinline__ void draft_phase2(const float (&x)[16], int vw, int khalf, int V, int wave,
                                             const float* wm /*[4][32] at lane*/, const int* wi, int lrow,
                                             float c, float* rec) {
  float M = wm[lrow];
  int I = wi[lrow];
#pragma unroll
  for (int w = 1; w < 4; ++w) amax_merge(M, I, wm[w * 32 + lrow], wi[w * 32 + lrow]);
  float e = 0.0f;
  if (c > 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = vw + acc_row(i, khalf);
      if (v < V) e += exp2_hw((x[i] - M) * c);
    }
  }
  const float eo = __shfl_xor(e, 32);
  const float tot = khalf ? (eo + e) : (e + eo);
  if (khalf == 0 && rec != nullptr) {
    if (wave == 0) {
      rec[0] = M;
      rec[1] = __int_as_float(I);
    }
    rec[2 + wave] = tot;
  }
}

// Residual epilogue: this wave's sum of max(0, p - q) for the lane's request.
__device__ __forceinline__ void resid_epilogue(const f32x16_t& acc, const float (&x)[16],
                                               const float* __restrict__ trow, int vw, int khalf, int V,
                                               bool vec4, bool ok, const ChunkInfo& ci, int wave,
                                               float* rec) {
  float t[16];
  load_row16(trow, vw + 4 * khalf, V, vec4, ok, t);
  float w = 0.0f;
  if (ok) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = vw + acc_row(i, khalf);
      if (v < V) {
        const float s = acc[i] + x[i];
        const float q = exp2_hw((s - ci.Mq) * ci.c) * ci.iZq;
        const float pp = exp2_hw((t[i] - ci.Mp) * ci.c) * ci.iZp;
        w += fmaxf(pp - q, 0.0f);
      }
    }
  }
  const float wo = __shfl_xor(w, 32);
  const float tot = khalf ? (wo + w) : (w + wo);
  if (khalf == 0 && ok && rec != nullptr) rec[2 + wave] = tot;
}

// ---------------------------------------------------------------------------
// bf16 weights: W2 fragments cached in registers for the whole kernel.
// KREG = number of 16-wide k steps held (rank <= 16 * KREG).
// ---------------------------------------------------------------------------
template <int KREG, bool RESID>
__global__ void __launch_bounds__(256) bias_tile_bf16(TileParams p) {
  constexpr int RS = KREG * 16 + 8;  // LDS row stride (bf16 elements): 16-byte pad vs bank conflicts
  __shared__ __attribute__((aligned(16))) uint16_t Hs[kNchBf16 * RS];
  __shared__ ChunkInfo s_ci[kNchBf16];
  __shared__ float s_wm[2][4 * 32];
  __shared__ int s_wi[2][4 * 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, khalf = lane >> 5;
  const int tile = blockIdx.x;
  const int vw = tile * kTileRows + wave * kSubRows;
  const int V = p.V, rank = p.rank, R = p.R;
  const bool vec4 = (V & 3) == 0;

  if (RESID) {
    int any = 0;
    for (int n = tid; n < R; n += 256) any |= p.rs_info[4 * static_cast<int64_t>(n)];
    if (!__syncthreads_or(any)) return;
  }

  // W2 rows of this wave as A fragments, all k.
  bf16x8_t wf[KREG];
  {
    const int v = vw + lrow;
    const uint16_t* w2 = static_cast<const uint16_t*>(p.W2) + static_cast<int64_t>(v < V ? v : 0) * rank;
#pragma unroll
    for (int ks = 0; ks < KREG; ++ks) {
      const int k0 = ks * 16 + khalf * 8;
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (v < V && k0 < rank) raw = *reinterpret_cast<const u32x4_t*>(w2 + k0);
      wf[ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  for (int n0 = 0; n0 < R; n0 += kNchBf16) {
    __syncthreads();  // previous chunk done with LDS
    if (tid < kNchBf16) s_ci[tid] = fetch_info(p, n0 + tid, RESID);
    __syncthreads();

    // H = W1[prev] rows of this chunk into LDS; k >= rank zero-filled.
    {
      constexpr int G = KREG * 2;
      const int gv = rank / 8;
      const uint16_t* w1 = static_cast<const uint16_t*>(p.W1);
      for (int q = tid; q < kNchBf16 * G; q += 256) {
        const int nn = q / G, g = q - nn * G;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (g < gv && s_ci[nn].act)
          val = *reinterpret_cast<const u32x4_t*>(w1 + static_cast<int64_t>(s_ci[nn].prev) * rank + g * 8);
        *reinterpret_cast<u32x4_t*>(&Hs[nn * RS + g * 8]) = val;
      }
    }

    // Base logits of this lane's rows for both column blocks.
    float x[2][16];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int nn = nb * 32 + lrow, n = n0 + nn;
      const ChunkInfo& ci = s_ci[nn];
      const bool ok = (n < R) && ci.act;
      const float* urow = RESID ? (p.U + static_cast<int64_t>(ci.urow) * V)
                                : (p.U_base + static_cast<int64_t>(ok ? n : 0) * p.U_stride);
      load_row16(urow, vw + 4 * khalf, V, vec4, ok, x[nb]);
    }
    __syncthreads();  // H ready

    f32x16_t acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc[nb] = f32x16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (n0 + nb * 32 < R) {
        const uint16_t* hrow = &Hs[(nb * 32 + lrow) * RS + khalf * 8];
#pragma unroll
        for (int ks = 0; ks < KREG; ++ks) {
          const u32x4_t braw = *reinterpret_cast<const u32x4_t*>(hrow + ks * 16);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], __builtin_bit_cast(bf16x8_t, braw),
                                                            acc[nb], 0, 0, 0);
        }
      }
    }

    if (!RESID) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        draft_phase1(acc[nb], x[nb], vw, khalf, V, &s_wm[nb][wave * 32 + lrow], &s_wi[nb][wave * 32 + lrow]);
      __syncthreads();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int nn = nb * 32 + lrow, n = n0 + nn;
        float* rec = (n < R) ? p.part + (static_cast<int64_t>(n) * p.n_tiles + tile) * kPartFloats : nullptr;
        draft_phase2(x[nb], vw, khalf, V, wave, s_wm[nb], s_wi[nb], lrow, s_ci[nn].c, rec);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int nn = nb * 32 + lrow, n = n0 + nn;
        const ChunkInfo ci = s_ci[nn];
        const bool ok = (n < R) && ci.act;
        float* rec = ok ? p.part + (static_cast<int64_t>(n) * p.n_tiles + tile) * kPartFloats : nullptr;
        resid_epilogue(acc[nb], x[nb], p.target + static_cast<int64_t>(ci.trow) * V, vw, khalf, V, vec4, ok,
                       ci, wave, rec);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 weights: v_mfma_f32_32x32x2_f32, W2 streamed from memory per k step.
// A lane l holds W2[row l&31][k = 2*ks + (l>>5)]; B the same k of H.
// ---------------------------------------------------------------------------
template <bool RESID>
__global__ void __launch_bounds__(256) bias_tile_f32(TileParams p) {
  constexpr int RS = DSPARK_MAX_RANK + 4;
  __shared__ __attribute__((aligned(16))) float Hf[kNchF32 * RS];
  __shared__ ChunkInfo s_ci[kNchF32];
  __shared__ float s_wm[4 * 32];
  __shared__ int s_wi[4 * 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, khalf = lane >> 5;
  const int tile = blockIdx.x;
  const int vw = tile * kTileRows + wave * kSubRows;
  const int V = p.V, rank = p.rank, R = p.R;
  const bool vec4 = (V & 3) == 0;

  if (RESID) {
    int any = 0;
    for (int n = tid; n < R; n += 256) any |= p.rs_info[4 * static_cast<int64_t>(n)];
    if (!__syncthreads_or(any)) return;
  }
  const int v_a = vw + lrow;
  const float* w2row = static_cast<const float*>(p.W2) + static_cast<int64_t>(v_a < V ? v_a : 0) * rank;

  for (int n0 = 0; n0 < R; n0 += kNchF32) {
    __syncthreads();
    if (tid < kNchF32) s_ci[tid] = fetch_info(p, n0 + tid, RESID);
    __syncthreads();
    {
      const float* w1 = static_cast<const float*>(p.W1);
      for (int q = tid; q < kNchF32 * rank; q += 256) {
        const int nn = q / rank, k = q - nn * rank;
        Hf[nn * RS + k] = s_ci[nn].act ? w1[static_cast<int64_t>(s_ci[nn].prev) * rank + k] : 0.0f;
      }
    }
    float x[16];
    {
      const int nn = lrow, n = n0 + nn;
      const ChunkInfo& ci = s_ci[nn];
      const bool ok = (n < R) && ci.act;
      const float* urow = RESID ? (p.U + static_cast<int64_t>(ci.urow) * V)
                                : (p.U_base + static_cast<int64_t>(ok ? n : 0) * p.U_stride);
      load_row16(urow, vw + 4 * khalf, V, vec4, ok, x);
    }
    __syncthreads();

    f32x16_t acc = f32x16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* hrow = &Hf[lrow * RS + khalf];
    for (int ks = 0; ks < rank / 2; ++ks) {
      const float a = (v_a < V) ? w2row[2 * ks + khalf] : 0.0f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, hrow[2 * ks], acc, 0, 0, 0);
    }

    const int n = n0 + lrow;
    if (!RESID) {
      draft_phase1(acc, x, vw, khalf, V, &s_wm[wave * 32 + lrow], &s_wi[wave * 32 + lrow]);
      __syncthreads();
      float* rec = (n < R) ? p.part + (static_cast<int64_t>(n) * p.n_tiles + tile) * kPartFloats : nullptr;
      draft_phase2(x, vw, khalf, V, wave, s_wm, s_wi, lrow, s_ci[lrow].c, rec);
    } else {
      const ChunkInfo ci = s_ci[lrow];
      const bool ok = (n < R) && ci.act;
      float* rec = ok ? p.part + (static_cast<int64_t>(n) * p.n_tiles + tile) * kPartFloats : nullptr;
      resid_epilogue(acc, x, p.target + static_cast<int64_t>(ci.trow) * V, vw, khalf, V, vec4, ok, ci, wave,
                     rec);
    }
  }
}

template <bool RESID>
hipError_t launch_bf16(const TileParams& p, hipStream_t s) {
  const dim3 grid(p.n_tiles), block(256);
  if (p.rank <= 64) {
    hipLaunchKernelGGL((bias_tile_bf16<4, RESID>), grid, block, 0, s, p);
  } else if (p.rank <= 128) {
    hipLaunchKernelGGL((bias_tile_bf16<8, RESID>), grid, block, 0, s, p);
  } else if (p.rank <= 256) {
    hipLaunchKernelGGL((bias_tile_bf16<16, RESID>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((bias_tile_bf16<32, RESID>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bias_tile(const TileParams& p, int wdtype, bool residual, hipStream_t s) {
  if (p.R == 0 || p.n_tiles == 0) return hipSuccess;
  if (wdtype == DSPARK_W_BF16) return residual ? launch_bf16<true>(p, s) : launch_bf16<false>(p, s);
  const dim3 grid(p.n_tiles), block(256);
  if (residual)
    hipLaunchKernelGGL((bias_tile_f32<true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((bias_tile_f32<false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
