// Fused Markov bias + softmax statistics over the vocabulary (gfx950).
//
// The Markov head's bias for request n is B[n, v] = sum_j W2[v, j] * W1[prev_n, j]
// ("DSpark" explainer, section 7; llama.cpp PR #25173 description:
// bias(prev) = markov_w2 . markov_w1[prev]).  For a batch of requests this is
// the product B^T = W2 . H^T with H = W1[prev] gathered row by row: W2 is
// streamed from HBM once per draft position as MFMA A fragments, H sits in
// LDS, and the epilogue adds the base logits U and reduces each request's
// values over a vocabulary segment (one wavefront's rows) in registers to one
// record of two floats.  Neither B nor s = U + B is ever written to memory,
// and no wavefront waits for another after the prologue.
//
//   draft record    (max_v s, sum_v exp((s_v - max)/T))  sampled request
//                   (max_v s, lowest argmax as int bits)  greedy request
//   residual record (0, sum_v max(0, p_v - q_v))
//
// Paths:
//   bias_seg16      bf16 weights, R <= 64.  v_mfma_f32_16x16x32_bf16; each
//                   wavefront owns 16-row segments; persistent workgroups
//                   (one per CU) gather H once and prefetch the next
//                   segment's W2 / U fragments while computing the current
//                   one.
//   bias_seg64      bf16 weights, R > 64.  v_mfma_f32_16x16x32_bf16; each
//                   wavefront keeps its 64 rows of W2 in registers while the
//                   requests stream through in chunks of 16 (H via LDS).
//   bias_seg32_f32  fp32 weights.  v_mfma_f32_32x32x2_f32.
//
// Operand layouts (wave64).  16x16x32: A lane l holds row (l & 15), 8 k at
// 8 * (l >> 4) of each 32-k step; B likewise for its column; accumulator i of
// lane l is row 4*(l>>4) + i, column (l & 15).  32x32x16: A lane l holds row
// (l & 31), 8 k at 8 * (l >> 5); accumulator i is row 8*(i/4) + 4*(l>>5) +
// (i%4), column (l & 31).  Rows are vocabulary entries, columns requests.

#include <hip/hip_ext.h>

#include "dspark_device.h"
#include "launchers.h"
#include "plan.h"

namespace dspark {
namespace {

// s_waitcnt immediate (gfx9 encoding): vmcnt 0, expcnt and lgkmcnt not waited for
constexpr int kVmcntZero = 0x0F70;

// LDS-only workgroup barrier: orders LDS traffic without draining the
// wavefront's outstanding global loads (a full __syncthreads() waits for
// every in-flight prefetch).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// Per-request values staged in LDS.
struct ReqInfo {
  int act, prev, urow, trow;
  float c, Mq, iZq, Mp, iZp;
};

// The rows a draft position reads: request n's previous token at
// prev_base[n * prev_stride], its base logits at U_base + n * U_stride.
struct Pos {
  const int32_t* prev_base;
  int prev_stride;
  const float* U_base;
  // RNN head: the fp32 states (draft: request n's row at h_base + n *
  // h_stride; residual: row urow of h_base)
  const float* h_base;
  int64_t h_stride;
};
__device__ __forceinline__ Pos pos_of(const TileParams& p) {
  return Pos{p.prev_base, p.prev_stride, p.U_base, p.h_base, p.h_stride};
}

// Every load is issued before the first value is used (the temperature's
// scale, computed under a branch, would otherwise hold back the others).
__device__ __forceinline__ ReqInfo fetch_info(const TileParams& p, const Pos& ps, int n, bool resid) {
  ReqInfo ci{0, 0, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n >= p.R) return ci;
  const float T = p.temp[n];
  if (!resid) {
    ci.act = 1;
    ci.prev = ps.prev_base[static_cast<int64_t>(n) * ps.prev_stride];
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
  ci.c = temp_scale(T);
  ci.prev = clampi(ci.prev, 0, p.V - 1);
  // rows of inactive requests are never used, but their loads are still
  // issued: keep every row index inside its buffer
  ci.urow = ci.act ? static_cast<int>(min(max(static_cast<int64_t>(ci.urow), int64_t{0}), p.u_rows - 1)) : 0;
  ci.trow = ci.act ? static_cast<int>(min(max(static_cast<int64_t>(ci.trow), int64_t{0}), p.t_rows - 1)) : 0;
  return ci;
}

__device__ __forceinline__ const float* u_row(const TileParams& p, const Pos& ps, const ReqInfo& ci, int n,
                                             bool resid) {
  return resid ? p.U + static_cast<int64_t>(ci.urow) * p.V : ps.U_base + static_cast<int64_t>(n) * p.U_stride;
}

// Four consecutive logits starting at v (clamped addresses; the caller masks).
template <bool VEC4>
__device__ __forceinline__ f32x4_t load4(const float* row, int v, int V) {
  if (VEC4) {
    return *reinterpret_cast<const f32x4_t*>(row + min(v, V - 4));
  } else {
    f32x4_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = row[min(v + e, V - 1)];
    return r;
  }
}

// ---------------------------------------------------------------------------
// 16-row path
// ---------------------------------------------------------------------------
// NB: request column blocks of 16 (1, 2 or 4: R <= 16, 32 or 64); the
// columns past the batch are not computed.
template <int KS, bool RESID, int NB>
struct Seg16Regs {
  bf16x8_t w[KS];     // W2 rows vw + (lane & 15), k = 32 ks + 8 (lane >> 4) .. +8
  f32x4_t u[NB];      // U[request 16 nb + (lane & 15)][vw + 4 (lane >> 4) .. +4]
  f32x4_t t[RESID ? NB : 1];  // target values, residual mode
};

// W2 fragment ks of segment [vw, vw + 16) for this lane: from the
// fragment-packed copy (1 KiB contiguous per k-step and wavefront; zeros
// past V and the rank), or from the row-major W2, where rows past V re-read
// row V - 1 and columns k >= rank re-read the row's last 8 weights (both
// masked at use).
// ASEG (the RNN head's draft mode): a segment past the vocabulary's holds
// rows vw - 16 n_seg .. +16 of A instead, in the same layout (rows past the
// rank re-read row rank - 1, or are zero in the packed copy; never stored).
template <int KS, bool PACKED, bool ASEG = false>
__device__ __forceinline__ const uint16_t* seg16_w2(const TileParams& p, int vw, int lane) {
  if (ASEG && vw >= p.n_seg * kSegSmall) {
    const int va = vw - p.n_seg * kSegSmall;
    if (PACKED) return p.ap + (static_cast<int64_t>(va / kSegSmall) * KS * 64 + lane) * 8;
    return p.A + static_cast<int64_t>(min(va + (lane & 15), p.rank - 1)) * p.rank;
  }
  if (PACKED) return p.w2p + (static_cast<int64_t>(vw / kSegSmall) * KS * 64 + lane) * 8;
  return static_cast<const uint16_t*>(p.W2) + static_cast<int64_t>(min(vw + (lane & 15), p.V - 1)) * p.rank;
}
template <int KS, bool PACKED>
__device__ __forceinline__ bf16x8_t seg16_w2_frag(const uint16_t* w2, int ks, int lane, int rank) {
  const uint16_t* a = PACKED ? w2 + ks * 512 : w2 + min(ks * 32 + (lane >> 4) * 8, rank - 8);
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(a));
}

// Issues the loads of segment [vw, vw + 16).  No instruction touches the
// loaded registers before the MFMA or the epilogue needs them (the rank and
// vocabulary masks are applied at use).
template <int KS, bool RESID, bool VEC4, bool PACKED, int NB, bool ASEG = false>
__device__ __forceinline__ void seg16_load(const TileParams& p, const Pos& ps, const ReqInfo* s_ci, int vw, int lane,
                                           Seg16Regs<KS, RESID, NB>& f) {
  const int l16 = lane & 15, kq = lane >> 4;
  const int V = p.V, rank = p.rank;
  const uint16_t* w2 = seg16_w2<KS, PACKED, ASEG>(p, vw, lane);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) f.w[ks] = seg16_w2_frag<KS, PACKED>(w2, ks, lane, rank);
  const int vu = vw + kq * 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nn = nb * 16 + l16;
    const ReqInfo& ci = s_ci[nn];
    f.u[nb] = load4<VEC4>(u_row(p, ps, ci, nn < p.R ? nn : 0, RESID), vu, V);
    if (RESID) f.t[nb] = load4<VEC4>(p.target + static_cast<int64_t>(ci.trow) * V, vu, V);
  }
}

// The segment's MFMAs (H from LDS), with the next segment's loads
// interleaved: k-step ks issues W2 fragment ks of segment [vw_next,
// vw_next + 16) (and, in the first steps, its U / target values), so a load
// issue that stalls on a busy memory pipeline holds up one k-step instead of
// a whole segment.  B (H) is read one k-step ahead when DBUF, else just in
// time (the draft kernel runs two wavefronts per SIMD, which cover the LDS
// latency, and needs the registers).  SPLIT: H is two bf16 planes (hi, lo:
// an fp32 state), and each k-step runs one MFMA per plane.
template <int KS, bool RESID, bool VEC4, bool DBUF, bool PACKED, int NB, bool SPLIT>
__device__ __forceinline__ void seg16_mfma_pf(const bf16x8_t (&w)[KS], const uint16_t* Hs, int rank, int lane,
                                              f32x4_t (&acc)[NB], const TileParams& p, const Pos& ps,
                                              const ReqInfo* s_ci, int vw_next, Seg16Regs<KS, RESID, NB>& nx) {
  constexpr int RS = KS * 32 + 8;
  constexpr int kPlane = NB * 16 * RS;  // offset of the lo plane (SPLIT)
  constexpr int NP = SPLIT ? 2 : 1;
  const int l16 = lane & 15, kq = lane >> 4;
  const int V = p.V;
  const uint16_t* w2n = seg16_w2<KS, PACKED, SPLIT && !RESID>(p, vw_next, lane);
  const int vu = vw_next + kq * 4;
  auto issue_u = [&](int nb) {
    const int nn = nb * 16 + l16;
    const ReqInfo& ci = s_ci[nn];
    nx.u[nb] = load4<VEC4>(u_row(p, ps, ci, nn < p.R ? nn : 0, RESID), vu, V);
    if (RESID) nx.t[nb] = load4<VEC4>(p.target + static_cast<int64_t>(ci.trow) * V, vu, V);
  };
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint16_t* h0 = Hs + l16 * RS + kq * 8;
  u32x4_t b[DBUF ? 2 : 1][NP][NB];
  if constexpr (DBUF) {
#pragma unroll
    for (int pl = 0; pl < NP; ++pl)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        b[0][pl][nb] = *reinterpret_cast<const u32x4_t*>(h0 + pl * kPlane + nb * 16 * RS);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    nx.w[ks] = seg16_w2_frag<KS, PACKED>(w2n, ks, lane, rank);
    if (ks < NB) issue_u(ks);
    const int cur = DBUF ? (ks & 1) : 0;
    if constexpr (DBUF) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int pl = 0; pl < NP; ++pl)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            b[cur ^ 1][pl][nb] =
                *reinterpret_cast<const u32x4_t*>(h0 + pl * kPlane + nb * 16 * RS + (ks + 1) * 32);
      }
    } else {
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          b[0][pl][nb] = *reinterpret_cast<const u32x4_t*>(h0 + pl * kPlane + nb * 16 * RS + ks * 32);
    }
    // the empty asm pins the zeroing here: hoisted next to the load (across
    // the loop's back edge) it would wait on the whole prefetch
    bf16x8_t a = w[ks];
    asm volatile("" : "+v"(a));
    a = (ks * 32 + kq * 8 < rank) ? a : bf16x8_t{};
#pragma unroll
    for (int pl = 0; pl < NP; ++pl)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, b[cur][pl][nb]), acc[nb],
                                                          0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int nb = KS; nb < NB; ++nb) issue_u(nb);  // fewer k-steps than U groups (rank <= 96)
}

// Per-lane copies of the request constants of the lane's NB requests
// (request 16 nb + (lane & 15)), kept in registers for the whole walk.
template <bool RESID, int NB>
struct LaneReq {
  float c[NB];  // log2(e) / T, 0 for greedy
  float Mq[RESID ? NB : 1], iZq[RESID ? NB : 1], Mp[RESID ? NB : 1], iZp[RESID ? NB : 1];
};

template <bool RESID, int NB>
__device__ __forceinline__ void lane_req(const ReqInfo* s_ci, int lane, LaneReq<RESID, NB>& q) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const ReqInfo ci = s_ci[nb * 16 + (lane & 15)];
    q.c[nb] = ci.c;
    if (RESID) {
      q.Mq[nb] = ci.Mq;
      q.iZq[nb] = ci.iZq;
      q.Mp[nb] = ci.Mp;
      q.iZp[nb] = ci.iZp;
    }
  }
}

// Epilogue of one 16-row segment, branch-free: reduces the 16 rows held by
// the four lanes (lane & 15) + 16 j of each request column and stores the
// segment's record.  All four lanes hold the reduced record and all store it
// (same value, same address); records of absent requests land in padding
// rows of the workspace and are never read.
template <int KS, bool RESID, int NB>
__device__ __forceinline__ void seg16_epilogue(const TileParams& p, const LaneReq<RESID, NB>& q, int wt, int lane,
                                               const Seg16Regs<KS, RESID, NB>& f, const f32x4_t (&acc)[NB]) {
  const int l16 = lane & 15, kq = lane >> 4;
  const int V = p.V;
  const int vb = wt * kSegSmall + kq * 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nn = nb * 16 + l16;
    const float c = q.c[nb];
    f32x4_t s = acc[nb] + f.u[nb];
    float x, y;
    if (!RESID) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (vb + i < V) ? s[i] : -INFINITY;
      float m = s[0];
      int im = vb;
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const bool gt = s[i] > m;
        m = gt ? s[i] : m;
        im = gt ? vb + i : im;
      }
      quad_amax(m, im);
      // exp2(-inf) = 0 for rows past V; a greedy request (c = 0) keeps im
      float e = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) e += exp2_rel(s[i], m, c);
      e = quad_sum(e);
      x = m;
      y = (c > 0.f) ? e : __int_as_float(im);
    } else {
      float w = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float qq = exp2_hw((s[i] - q.Mq[nb]) * c) * q.iZq[nb];
        const float pp = exp2_hw((f.t[nb][i] - q.Mp[nb]) * c) * q.iZp[nb];
        // rows past V add +0 (a bit mask, not a branch around the exps)
        const float d = fmaxf(pp - qq, 0.f);
        w += __int_as_float(__float_as_int(d) & -static_cast<int>(vb + i < V));
      }
      w = quad_sum(w);
      x = 0.f;
      y = w;
    }
    float2* rec = reinterpret_cast<float2*>(p.part) + static_cast<int64_t>(nn) * p.n_seg + wt;
    *rec = make_float2(x, y);
  }
}

// RNN head, draft mode: the segment wt >= n_seg holds rows (wt - n_seg) * 16
// .. +16 of A; z = A h of request 16 nb + (lane & 15), rows 4 (lane >> 4)
// .. +4 of the segment, stored as fp32 for the next state (rows past the
// rank and absent requests are not stored).
template <int NB>
__device__ __forceinline__ void seg16_store_z(const TileParams& p, int wt, int lane, const f32x4_t (&acc)[NB]) {
  const int l16 = lane & 15, kq = lane >> 4;
  const int j0 = (wt - p.n_seg) * kSegSmall + kq * 4;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nn = nb * 16 + l16;
    if (nn < p.R) {
      float* z = p.z_out + static_cast<int64_t>(nn) * p.h_stride;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + i < p.rank) z[j0 + i] = acc[nb][i];
    }
  }
}

constexpr int kSeg16Waves = 4;     // residual mode: wavefronts per workgroup, one per SIMD
constexpr int kSeg16DraftWaves = 8;  // draft mode: one workgroup per CU, two wavefronts per SIMD
constexpr int kSeg16GatherWaves = 4;  // draft mode: wavefronts that gather H

// H of the RNN head: request nn's fp32 state row (draft mode: h_base +
// nn * h_stride; residual mode: row urow of h_base, stride rank) split into
// a hi plane bf16(h) and a lo plane bf16(h - hi).  The states are stored as
// double-bf16 values (rnn.hip), so hi + lo == h exactly and the two MFMAs
// per k-step compute W2 h with exact products.
// Rows of inactive requests and groups past the rank are zero.  The caller
// has stored the request info (s_ci) and passed a barrier.
template <int KS, bool RESID, int GW, int NB>
__device__ __forceinline__ void seg16_state_h(const TileParams& p, const Pos& ps, uint16_t* Hs,
                                              const ReqInfo* s_ci) {
  constexpr int RS = KS * 32 + 8;
  constexpr int G = KS * 4;
  constexpr int kPieces = NB * 16 * G;
  constexpr int kPer = (kPieces + GW * 64 - 1) / (GW * 64);
  constexpr int kPlane = NB * 16 * RS;
  const int tid = threadIdx.x;
  const int rank = p.rank;
  if (tid >= GW * 64) {
    lds_barrier();
    return;
  }
  f32x4_t va[kPer], vb[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = min(tid + j * GW * 64, kPieces - 1);
    const int nn = q / G, g = q - nn * G;
    const int64_t row = RESID ? static_cast<int64_t>(s_ci[nn].urow) * rank
                              : static_cast<int64_t>(nn < p.R ? nn : 0) * ps.h_stride;
    const float* h = ps.h_base + row + min(g * 8, rank - 8);
    va[j] = *reinterpret_cast<const f32x4_t*>(h);
    vb[j] = *reinterpret_cast<const f32x4_t*>(h + 4);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + j * GW * 64;
    const int nn = q / G, g = q - nn * G;
    const bool zero = g * 8 >= rank || !s_ci[nn].act;
    u32x4_t hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = e < 2 ? va[j][2 * e] : vb[j][2 * e - 4];
      const float x1 = e < 2 ? va[j][2 * e + 1] : vb[j][2 * e - 3];
      const uint32_t h0 = bf16_rne_bits(x0), h1 = bf16_rne_bits(x1);
      const uint32_t l0 = bf16_rne_bits(x0 - __uint_as_float(h0 << 16));
      const uint32_t l1 = bf16_rne_bits(x1 - __uint_as_float(h1 << 16));
      hi[e] = zero ? 0u : (h0 | (h1 << 16));
      lo[e] = zero ? 0u : (l0 | (l1 << 16));
    }
    if (kPieces % (GW * 64) == 0 || q < kPieces) {
      *reinterpret_cast<u32x4_t*>(&Hs[nn * RS + g * 8]) = hi;
      *reinterpret_cast<u32x4_t*>(&Hs[kPlane + nn * RS + g * 8]) = lo;
    }
  }
  lds_barrier();
}

// Request info and H = W1[prev] for all requests of the 16-row path, into
// LDS (the workgroup's first barrier comes after the info, the second after
// H).  The info is read by wavefront 0 and H by the first GW wavefronts;
// every 16-byte load of a thread is issued before any is stored.
template <int KS, bool RESID, int GW, int NB, bool SPLIT>
__device__ __forceinline__ void seg16_info_h(const TileParams& p, const Pos& ps, uint16_t* Hs, ReqInfo* s_ci) {
  constexpr int RS = KS * 32 + 8;  // LDS row stride of H (bf16): 16-byte pad vs bank conflicts
  constexpr int G = KS * 4;        // 16-byte groups per H row
  constexpr int kPieces = NB * 16 * G;  // 16-byte pieces of the NB * 16 H rows
  constexpr int kPer = (kPieces + GW * 64 - 1) / (GW * 64);
  const int tid = threadIdx.x;
  const int rank = p.rank;
  if (tid < kSmallMaxR) s_ci[tid] = fetch_info(p, ps, tid, RESID);
  lds_barrier();
  if constexpr (SPLIT) {
    seg16_state_h<KS, RESID, GW, NB>(p, ps, Hs, s_ci);
    return;
  }
  if (tid >= GW * 64) {
    lds_barrier();
    return;
  }
  u32x4_t val[kPer];
  const uint16_t* w1 = static_cast<const uint16_t*>(p.W1);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = min(tid + j * GW * 64, kPieces - 1);
    const int nn = q / G, g = q - nn * G;
    val[j] = *reinterpret_cast<const u32x4_t*>(w1 + static_cast<int64_t>(s_ci[nn].prev) * rank + min(g * 8, rank - 8));
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + j * GW * 64;
    const int nn = q / G, g = q - nn * G;
    const u32x4_t v = (g * 8 >= rank || !s_ci[nn].act) ? u32x4_t{0u, 0u, 0u, 0u} : val[j];
    if (kPieces % (GW * 64) == 0 || q < kPieces) *reinterpret_cast<u32x4_t*>(&Hs[nn * RS + g * 8]) = v;
  }
  lds_barrier();
}

// The segments are dealt out in rounds of W = all wavefronts: round j is the
// contiguous stretch [j W, (j + 1) W), so at any moment the grid streams one
// stretch of W2 and of every U row (DRAM pages are read whole instead of 64
// bytes from each of 64 rows).  Workgroup b owns the WPB segments
// j W + b WPB + [0, WPB) of every round, in ticket order t = j WPB + i.  Its
// wavefront i starts on ticket i and then takes the next free ticket of the
// workgroup from an LDS counter, so a wavefront that streams faster takes
// more of its workgroup's segments instead of waiting at the end.  `fa`
// holds the loads of the wavefront's first segment sg, already issued; H
// and the request info are in LDS, and *ctr (LDS) was set to WPB before the
// last barrier.
template <int KS, bool RESID, bool VEC4, bool PACKED, int NB, bool SPLIT, int WPB>
__device__ __forceinline__ void seg16_walk(const TileParams& p, const Pos& ps, const uint16_t* Hs,
                                           const ReqInfo* s_ci, int sg, Seg16Regs<KS, RESID, NB>& fa,
                                           Seg16Regs<KS, RESID, NB>& fb, int* ctr) {
  constexpr bool DBUF = RESID;  // see seg16_mfma
  constexpr bool ASEG = SPLIT && !RESID;
  const int lane = threadIdx.x & 63;
  const int rank = p.rank, n_seg = p.n_seg;
  const int n_walk = ASEG ? n_seg + p.n_seg_a : n_seg;  // with the RNN head's A segments
  const int n_waves = gridDim.x * WPB;
  if (sg >= n_walk) return;
  LaneReq<RESID, NB> lq;
  lane_req<RESID, NB>(s_ci, lane, lq);
  // the segment of the workgroup's next free ticket (segments grow with the
  // ticket, so once one is past n_seg every later one is too)
  auto take = [&]() {
    int t = 0;
    if (lane == 0) t = atomicAdd(ctr, 1);
    t = __builtin_amdgcn_readfirstlane(t);
    return static_cast<int>(blockIdx.x) * WPB + (t % WPB) + (t / WPB) * n_waves;
  };
  // Ping-pong prefetch, the next segment's loads interleaved with the
  // current one's k-steps.  The prefetch issued on a wavefront's last
  // segment re-reads segment n_seg - 1 (a cache hit, never used) so that the
  // load stream, and with it the compiler's wait counts, is the same every
  // trip.
  auto finish = [&](int wt, const Seg16Regs<KS, RESID, NB>& f, const f32x4_t (&acc)[NB]) {
    if (ASEG && wt >= n_seg)
      seg16_store_z<NB>(p, wt, lane, acc);
    else
      seg16_epilogue<KS, RESID, NB>(p, lq, wt, lane, f, acc);
  };
  while (true) {
    f32x4_t acc[NB];
    const int s1 = take();
    seg16_mfma_pf<KS, RESID, VEC4, DBUF, PACKED, NB, SPLIT>(fa.w, Hs, rank, lane, acc, p, ps, s_ci,
                                                 min(s1, n_walk - 1) * kSegSmall, fb);
    finish(sg, fa, acc);
    if (s1 >= n_walk) break;
    const int s2 = take();
    seg16_mfma_pf<KS, RESID, VEC4, DBUF, PACKED, NB, SPLIT>(fb.w, Hs, rank, lane, acc, p, ps, s_ci,
                                                 min(s2, n_walk - 1) * kSegSmall, fa);
    finish(s1, fb, acc);
    if (s2 >= n_walk) break;
    sg = s2;
  }
}

template <int KS, bool RESID, bool VEC4, int WPB, bool PACKED, int NB, bool SPLIT>
__device__ __forceinline__ void bias_seg16_body(const TileParams& p, uint16_t* Hs, ReqInfo* s_ci, int* ctr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = p.R, n_seg = p.n_seg;
  if (tid == 0) *ctr = WPB;  // published by the barriers of seg16_info_h
  if (RESID) {
    int any = 0;
    for (int n = tid; n < R; n += WPB * 64) any |= p.rs_info[4 * static_cast<int64_t>(n)];
    if (!__syncthreads_or(any)) return;
  }
  // wavefront-uniform walk state (scalar registers, scalar branches)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int sg = blockIdx.x * WPB + wv;
  Seg16Regs<KS, RESID, NB> fa, fb;
  const Pos ps = pos_of(p);
  // draft mode: the first segment's W2 and U addresses depend on neither H
  // nor the request info, so the wavefronts that do not gather H issue its
  // loads first, and they are in flight while the request info and the H
  // rows (prev -> W1[prev]) arrive.  The gathering wavefronts issue theirs
  // after H: a wavefront's loads complete in issue order, so H loads queued
  // behind a segment's would wait for the segment.  The RNN head's fp32
  // states (twice the bytes of W1 rows) are gathered by every wavefront.
  constexpr int GW = (RESID || SPLIT) ? WPB : kSeg16GatherWaves;
  const bool early = !RESID && wv >= GW;
  constexpr bool ASEG = SPLIT && !RESID;
  const int vw0 = min(sg, n_seg + (ASEG ? p.n_seg_a : 0) - 1) * kSegSmall;
  if (early) seg16_load<KS, RESID, VEC4, PACKED, NB, ASEG>(p, ps, s_ci, vw0, lane, fa);
  seg16_info_h<KS, RESID, GW, NB, SPLIT>(p, ps, Hs, s_ci);
  // residual mode: the first segment's loads come after the barrier (their
  // U and target rows come from the request info)
  if (!early) seg16_load<KS, RESID, VEC4, PACKED, NB, ASEG>(p, ps, s_ci, vw0, lane, fa);
  seg16_walk<KS, RESID, VEC4, PACKED, NB, SPLIT, WPB>(p, ps, Hs, s_ci, sg, fa, fb, ctr);
}

// Draft mode: one workgroup of eight wavefronts per CU (two per SIMD, for
// latency hiding, sharing one copy of H); compiled to fit 256 registers per
// wavefront.
template <int KS, bool VEC4, bool PACKED, int NB, bool SPLIT>
__global__ void __launch_bounds__(kSeg16DraftWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bias_seg16(TileParams p) {
  constexpr int RS = KS * 32 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Hs[(SPLIT ? 2 : 1) * NB * 16 * RS];
  __shared__ ReqInfo s_ci[kSmallMaxR];
  __shared__ int ctr;
  bias_seg16_body<KS, false, VEC4, kSeg16DraftWaves, PACKED, NB, SPLIT>(p, Hs, s_ci, &ctr);
}

// Residual mode (holds the target values too): one wavefront per SIMD.
template <int KS, bool VEC4, bool PACKED, int NB, bool SPLIT>
__global__ void __launch_bounds__(kSeg16Waves * 64) bias_seg16_res(TileParams p) {
  constexpr int RS = KS * 32 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Hs[(SPLIT ? 2 : 1) * NB * 16 * RS];
  __shared__ ReqInfo s_ci[kSmallMaxR];
  __shared__ int ctr;
  bias_seg16_body<KS, true, VEC4, kSeg16Waves, PACKED, NB, SPLIT>(p, Hs, s_ci, &ctr);
}

// ---------------------------------------------------------------------------
// 64-row path (bf16 weights, R > 64): the product is a real GEMM
// ---------------------------------------------------------------------------
// A workgroup of four wavefronts owns 256 vocabulary rows; wavefront w keeps
// W2 rows [64 (4 blockIdx + w), +64) in registers for the whole launch, as
// four 16-row MFMA A blocks, so that every B fragment read from LDS feeds
// four MFMAs.  The requests stream through in chunks of 16 (one MFMA column
// block): while chunk c computes, the W1 rows of chunk c + 2 and the U (and
// target) values of chunk c + 2 are in flight in registers; H goes through a
// two-stage LDS ring with one barrier per chunk.  Per-request values come
// from an LDS window of 256 requests, loaded 16 chunks ahead.  Residual mode
// visits only the requests listed by verify_finish.
constexpr int kWideWin = 256;                          // requests per window (one per thread)
constexpr int kWideWinChunks = kWideWin / kWideChunk;  // chunks per window

template <bool RESID>
struct WideReq;
template <>
struct WideReq<false> {
  int n, prev;  // record row, previous token
  float c;      // log2(e) / T, 0 for greedy
};
template <>
struct WideReq<true> {
  int n, prev, urow, trow;
  float c, Mq, iZq, Mp, iZp;
};

// A request's raw inputs, held in registers between the window's load and
// its store into LDS (every derived value is computed at the store, so no
// instruction touches the loads early).
template <bool RESID>
struct WideRaw;
template <>
struct WideRaw<false> {
  int prev;
  float T;
};
template <>
struct WideRaw<true> {
  u32x4_t a, b;  // (n, prev, U row, target row), (Mq, Zq, Mp, Zp) of one ResidualEntry
  float T;
};

template <bool RESID>
__device__ __forceinline__ void wide_raw_load(const TileParams& p, int i, int cnt, WideRaw<RESID>& r) {
  const int j = min(i, cnt - 1);
  if constexpr (!RESID) {
    r.prev = p.prev_base[static_cast<int64_t>(j) * p.prev_stride];
    r.T = p.temp[j];
  } else {
    const u32x4_t* e = reinterpret_cast<const u32x4_t*>(p.rs_list + j);
    r.a = e[0];
    r.b = e[1];
    r.T = p.rs_list[j].T;
  }
}

template <bool RESID>
__device__ __forceinline__ void wide_raw_store(const TileParams& p, int i, int cnt, const WideRaw<RESID>& r,
                                               WideReq<RESID>& q) {
  // slots past the last request write their records into padding rows
  const int pad_row = p.R + (i & (kWideChunk - 1));
  if constexpr (!RESID) {
    q.n = (i < cnt) ? i : pad_row;
    q.prev = clampi(r.prev, 0, p.V - 1);
    q.c = temp_scale(r.T);
  } else {
    q.n = (i < cnt) ? clampi(static_cast<int>(r.a[0]), 0, p.R - 1) : pad_row;
    q.prev = clampi(static_cast<int>(r.a[1]), 0, p.V - 1);
    q.urow = static_cast<int>(min(max(static_cast<int64_t>(static_cast<int>(r.a[2])), int64_t{0}), p.u_rows - 1));
    q.trow = static_cast<int>(min(max(static_cast<int64_t>(static_cast<int>(r.a[3])), int64_t{0}), p.t_rows - 1));
    q.c = temp_scale(r.T);
    q.Mq = __uint_as_float(r.b[0]);
    q.iZq = 1.0f / __uint_as_float(r.b[1]);
    q.Mp = __uint_as_float(r.b[2]);
    q.iZp = 1.0f / __uint_as_float(r.b[3]);
  }
}

// W1 rows of one chunk in flight: 16-byte piece q = tid + 256 j is group
// q % (4 KS) of row q / (4 KS); pieces past the 16 rows go to a dummy row.
template <int KS>
struct WideH {
  static constexpr int kGroups = 4 * KS;  // 16-byte groups per LDS row
  static constexpr int kPer = (kWideChunk * kGroups + 255) / 256;
  u32x4_t v[kPer];
};

template <int KS, bool RESID>
__device__ __forceinline__ void wide_h_issue(const TileParams& p, const WideReq<RESID>* win, int cw, WideH<KS>& h) {
  constexpr int G = WideH<KS>::kGroups;
  const uint16_t* w1 = static_cast<const uint16_t*>(p.W1);
#pragma unroll
  for (int j = 0; j < WideH<KS>::kPer; ++j) {
    const int q = static_cast<int>(threadIdx.x) + j * 256;
    const int r = min(q / G, kWideChunk - 1), g = q % G;
    const int prev = win[cw * kWideChunk + r].prev;
    h.v[j] = *reinterpret_cast<const u32x4_t*>(w1 + static_cast<int64_t>(prev) * p.rank + min(g * 8, p.rank - 8));
  }
}

// Stores a chunk's W1 rows into an LDS stage; pieces past the 16 rows land
// in row 16.  Groups past the rank are not stored: wide_h_zero_tail clears
// them once in both stages, and they stay zero.  Their loads were clamped to
// the row's last real weights, and so were those of the W2 fragments, which
// are zeroed (wide_w2_ready) only in the last k-step, while a rank whose
// next-to-last k-step is not full (e.g. 72, 200 or 384) has such groups in
// earlier k-steps too.
template <int KS>
__device__ __forceinline__ void wide_h_commit(const WideH<KS>& h, int rank, uint16_t* stage) {
  constexpr int G = WideH<KS>::kGroups;
  constexpr int RS = KS * 32 + 8;
#pragma unroll
  for (int j = 0; j < WideH<KS>::kPer; ++j) {
    const int q = static_cast<int>(threadIdx.x) + j * 256;
    const int r = min(q / G, kWideChunk), g = q % G;
    if (g * 8 < rank) *reinterpret_cast<u32x4_t*>(stage + r * RS + g * 8) = h.v[j];
  }
}

// Zeroes the groups past the rank in every row of the nst LDS stages of
// kStage elements (no barrier).
template <int KS>
__device__ __forceinline__ void wide_h_zero_tail(int rank, uint16_t* Hs, int nst) {
  constexpr int G = WideH<KS>::kGroups;
  constexpr int RS = KS * 32 + 8;
  constexpr int kRows = kWideChunk + 1;
  for (int q = static_cast<int>(threadIdx.x); q < nst * kRows * G; q += 256) {
    const int row = q / G, g = q % G;  // row counts over the stages: stage st holds rows st * kRows ..
    if (g * 8 >= rank) *reinterpret_cast<u32x4_t*>(Hs + row * RS + g * 8) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Epilogue inputs of one chunk for this lane's request (16 c + (lane & 15)):
// U (and target) values of rows vw + 16 b + 4 (lane >> 4) .. +4, b < 4.
template <bool RESID>
struct WideU {
  f32x4_t u[4];
  f32x4_t t[RESID ? 4 : 1];
  int n;
  float c;
  float Mq, iZq, Mp, iZp;  // residual mode
};

template <bool RESID, bool VEC4>
__device__ __forceinline__ void wide_u_issue(const TileParams& p, const WideReq<RESID>* win, int chunk, int cw,
                                             int vw, int lane, WideU<RESID>& f) {
  const int l16 = lane & 15, kq = lane >> 4;
  const WideReq<RESID>& q = win[cw * kWideChunk + l16];
  f.n = q.n;
  f.c = q.c;
  const float* urow;
  if constexpr (!RESID) {
    urow = p.U_base + static_cast<int64_t>(min(chunk * kWideChunk + l16, p.R - 1)) * p.U_stride;
  } else {
    urow = p.U + static_cast<int64_t>(q.urow) * p.V;
    f.Mq = q.Mq;
    f.iZq = q.iZq;
    f.Mp = q.Mp;
    f.iZp = q.iZp;
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) f.u[b] = load4<VEC4>(urow, vw + 16 * b + 4 * kq, p.V);
  if constexpr (RESID) {
    const float* trow = p.target + static_cast<int64_t>(q.trow) * p.V;
#pragma unroll
    for (int b = 0; b < 4; ++b) f.t[b] = load4<VEC4>(trow, vw + 16 * b + 4 * kq, p.V);
  }
}

// Rows past the vocabulary become -inf (in U, and in the target values in
// residual mode), so that the logits and the exponentials of those rows
// need no per-row test.  `full` (the segment lies inside the vocabulary)
// is wavefront-uniform: only the wavefront whose segment holds row V - 1
// (or lies past it) runs the selects.
__device__ __forceinline__ void wide_mask(bool full, int vw, int lane, int V, f32x4_t (&x)[4]) {
  if (full) return;
  const int vb = vw + 4 * (lane >> 4);
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[b][i] = (vb + 16 * b + i < V) ? x[b][i] : -INFINITY;
}

// This wavefront's W2 rows vw + 16 b + (lane & 15), k = 32 ks + 8 (lane >> 4)
// .. +8, the MFMA A fragments (addresses clamped into the row; the groups
// past the rank are zeroed by wide_w2_ready).
template <int KS>
__device__ __forceinline__ void wide_w2_load(const TileParams& p, int vw, int lane, u32x4_t (&w)[4][KS]) {
  const int l16 = lane & 15, kq = lane >> 4;
  const uint16_t* w2 = static_cast<const uint16_t*>(p.W2);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int v = min(vw + 16 * b + l16, p.V - 1);
      w[b][ks] = *reinterpret_cast<const u32x4_t*>(w2 + static_cast<int64_t>(v) * p.rank +
                                                   min(ks * 32 + kq * 8, p.rank - 8));
    }
}

// Called once the prologue's other loads are issued: zeroes the groups past
// the rank in the last k-step (the H rows are zero in every group past the
// rank, wide_h_commit) and pins every fragment to the
// accumulation registers, the operand form the MFMA reads directly, which
// leaves the architectural registers to the stream.
template <int KS>
__device__ __forceinline__ void wide_w2_ready(int rank, int lane, u32x4_t (&w)[4][KS]) {
  const bool past = (KS - 1) * 32 + (lane >> 4) * 8 >= rank;
#pragma unroll
  for (int b = 0; b < 4; ++b) w[b][KS - 1] = past ? u32x4_t{0u, 0u, 0u, 0u} : w[b][KS - 1];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int b = 0; b < 4; ++b) asm volatile("" : "+a"(w[b][ks]));
}

// Base of the exponentials of a 64-row record: its maximum, or 0 when every
// row is masked (-inf), so that no entry computes -inf - (-inf).  A wholly
// masked segment then records the sum 0; its weight 2^((max - M) / T) in
// any finite-maximum total is 0 either way.  (A greedy request's sum is
// never used.)
__device__ __forceinline__ float wide_exp_base(float m) { return (m == -INFINITY) ? 0.f : m; }

// Residual-mode record of one chunk for this lane's request over the
// wavefront's 64 rows, cut into small steps placed between the MFMAs of the
// next chunk (step t is a compile-time constant at every call): step 3 k
// adds entry k of max(0, p - q) (the two steps after it are empty), step 48
// combines the four lanes (lane & 15) + 16 j and stores.  The accumulators
// start at zero: the bf16 products are exact in fp32 and their partial sums
// stay exactly representable, so the bias W2 h comes out exact in any
// summation order, and s = bias + U is the value every other pass over the
// same row computes bit for bit.
constexpr int kEpiSteps = 49;

struct WideEpi {
  float z;
  int n;
};

__device__ __forceinline__ void wide_resid_step(int t, const TileParams& p, int seg, bool full, int lane,
                                                WideU<true>& f, const f32x4_t (&acc)[4], bool live, WideEpi& e) {
  if (t < 48 && t % 3 == 0) {
    const int k = t / 3, b = k >> 2, i = k & 3;
    if (k == 0) {
      e.z = 0.f;
      e.n = f.n;
      wide_mask(full, seg * kSegWide, lane, p.V, f.u);
      wide_mask(full, seg * kSegWide, lane, p.V, f.t);
    }
    const float qq = exp2_hw((acc[b][i] + f.u[b][i] - f.Mq) * f.c) * f.iZq;
    const float pp = exp2_hw((f.t[b][i] - f.Mp) * f.c) * f.iZp;
    e.z += fmaxf(pp - qq, 0.f);
  } else if (t == 48) {
    const float z = quad_sum(e.z);
    const bool in_v = live && seg < p.n_seg;
    const int64_t row = in_v ? e.n : p.R + kWideChunk;
    const int col = in_v ? seg : 0;
    reinterpret_cast<float2*>(p.part)[row * p.n_seg + col] = make_float2(0.f, z);
  }
}

// Draft-mode record of one chunk (the maximum over the wavefront's 64 rows
// for this lane's request, and its lowest argmax or the sum of
// 2^((s - max) c)) as fixed work per sub-slot: sub-slot j runs right after
// MFMA j of the next chunk (one sub-slot per MFMA at rank 512), with no
// branch besides the rare vocabulary mask, so that the scheduler keeps every
// piece where it is put.  Rows past V are -inf through U; the exponentials
// use the maximum as base (0 when all 64 rows are masked, wide_exp_base).
// One wavefront per SIMD does not overlap its own vector work with its
// MFMAs, but work spread this way waits on no result of the last few
// instructions, while the same work gathered into runs stalls on each
// dependent step.  Every lane computes both the lowest argmax and the
// exponential sum (a chunk's requests may be greedy and sampled at once).
// Each piece reads only results of earlier sub-slots:
//   3-10   logits s_k = acc + U, two per sub-slot; 4-11 the lane maximum
//   12-20  lowest index of the maximum, scanning down: compares one sub-slot
//          ahead of their selects
//   21-26  (max, lowest argmax) over the four lanes (lane & 15) + 16 j
//   27-45  z = sum of 2^((s_k - max) c), in index order (sub-slot n + 28
//          forms exponent k = n, n + 29 takes its power, n + 30 adds it)
//   46-49  sum over the four lanes; 50 stores (max, sum) or (max, argmax)
// The epilogue inputs are free after sub-slot 11 (the next chunk's may be
// loaded into them from sub-slot 12 on).
constexpr int kDraftUFree = 12;
constexpr int kDraftEpiEnd = 51;

struct WideDraftEpi {
  float s[16];
  float m, mg, z, c, tt[2], ee[2];
  uint32_t ml, mh, il, ih;
  int im, n;
  bool eq0, eq1, take;
};

__device__ __forceinline__ void wide_draft_slot(int j, const TileParams& p, int seg, bool full, int lane,
                                                WideU<false>& f, const f32x4_t (&acc)[4], bool live,
                                                WideDraftEpi& e) {
  const int vb = seg * kSegWide + 4 * (lane >> 4);
  auto row = [&](int k) { return vb + 16 * (k >> 2) + (k & 3); };
  if (j == 3) {
    e.c = f.c;
    e.n = f.n;
    wide_mask(full, seg * kSegWide, lane, p.V, f.u);
  }
  if (j >= 3 && j <= 10) {
    const int k = 2 * (j - 3);
    e.s[k] = acc[k >> 2][k & 3] + f.u[k >> 2][k & 3];
    e.s[k + 1] = acc[(k + 1) >> 2][(k + 1) & 3] + f.u[(k + 1) >> 2][(k + 1) & 3];
  }
  if (j == 4) e.m = fmaxf(e.s[0], e.s[1]);
  if (j >= 5 && j <= 11) {
    const int k = 2 * (j - 4);
    e.m = fmaxf(fmaxf(e.m, e.s[k]), e.s[k + 1]);
  }
  if (j >= 13 && j <= 20) {
    const int k = 15 - 2 * (j - 13);
    e.im = e.eq0 ? row(k) : e.im;
    e.im = e.eq1 ? row(k - 1) : e.im;
  }
  if (j == 12) e.im = kIntMax;
  if (j >= 12 && j <= 19) {
    const int k = 15 - 2 * (j - 12);
    e.eq0 = e.s[k] == e.m;
    e.eq1 = e.s[k - 1] == e.m;
  }
  if (j == 21 || j == 24) {
    if (j == 21) {
      lane_pair16(__float_as_uint(e.m), e.ml, e.mh);
      lane_pair16(static_cast<uint32_t>(e.im), e.il, e.ih);
    } else {
      lane_pair32(__float_as_uint(e.m), e.ml, e.mh);
      lane_pair32(static_cast<uint32_t>(e.im), e.il, e.ih);
    }
  }
  if (j == 22 || j == 25)
    e.take = amax_takes(__uint_as_float(e.mh), static_cast<int>(e.ih), __uint_as_float(e.ml), static_cast<int>(e.il));
  if (j == 23 || j == 26) {
    e.m = __uint_as_float(e.take ? e.mh : e.ml);
    e.im = static_cast<int>(e.take ? e.ih : e.il);
  }
  if (j == 27) {
    e.mg = wide_exp_base(e.m);
    e.z = 0.f;
  }
  if (j >= 28 && j <= 45) {
    const int n = j - 28;
    if (n >= 2) e.z += e.ee[n & 1];
    if (n >= 1 && n <= 16) e.ee[(n - 1) & 1] = exp2_hw(e.tt[(n - 1) & 1]);
    if (n < 16) e.tt[n & 1] = (e.s[n] - e.mg) * e.c;
  }
  if (j == 46) lane_pair16(__float_as_uint(e.z), e.ml, e.mh);
  if (j == 48) lane_pair32(__float_as_uint(e.z), e.ml, e.mh);
  if (j == 47 || j == 49) e.z = __uint_as_float(e.ml) + __uint_as_float(e.mh);
  if (j == 50) {
    const bool in_v = live && seg < p.n_seg;
    const int64_t r = in_v ? e.n : p.R + kWideChunk;
    const int col = in_v ? seg : 0;
    reinterpret_cast<float2*>(p.part)[r * p.n_seg + col] =
        make_float2(e.m, (e.c > 0.f) ? e.z : __int_as_float(e.im));
  }
}

template <int KS, bool RESID, bool VEC4>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) bias_seg64(TileParams p) {
  constexpr int RS = KS * 32 + 8;
  constexpr int kStage = (kWideChunk + 1) * RS;  // 16 rows + the dummy row
  __shared__ __attribute__((aligned(16))) uint16_t Hs[2 * kStage];
  __shared__ WideReq<RESID> win[2][kWideWin];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cnt = RESID ? min(max(p.rs_count[0], 0), p.R) : p.R;
  if (cnt == 0) return;
  const int n_chunks = (cnt + kWideChunk - 1) / kWideChunk;
  const int n_win = (n_chunks + kWideWinChunks - 1) / kWideWinChunks;
  const int seg = blockIdx.x * 4 + wave;
  const int vw = seg * kSegWide;
  const bool full = vw + kSegWide <= p.V;  // wavefront-uniform
  const int rank = p.rank;

  // window 0 (its loads are waited for at once: nothing else is in flight yet)
  WideRaw<RESID> raw;
  wide_raw_load<RESID>(p, tid, cnt, raw);
  wide_raw_store<RESID>(p, tid, cnt, raw, win[0][tid]);
  lds_barrier();
  // the first two chunks' W1 rows, then this wavefront's W2 rows, then the
  // first chunk's U values (the first H wait does not wait for W2)
  WideH<KS> h0, h1;
  wide_h_issue<KS, RESID>(p, win[0], 0, h0);
  wide_h_issue<KS, RESID>(p, win[0], min(1, n_chunks - 1), h1);
  u32x4_t w[4][KS];
  wide_w2_load<KS>(p, vw, lane, w);
  // ua / ub: epilogue inputs of the odd / even chunks; ua starts empty (the
  // first iteration's epilogue has no chunk: it stores into the dummy row)
  WideU<RESID> ua, ub;
  ua.n = 0;
  ua.c = 0.f;
  ua.Mq = ua.iZq = ua.Mp = ua.iZp = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) ua.u[b] = ua.t[RESID ? b : 0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  wide_u_issue<RESID, VEC4>(p, win[0], 0, 0, vw, lane, ub);
  wide_h_zero_tail<KS>(rank, Hs, 2);
  wide_h_commit<KS>(h0, rank, Hs);
  // every load of the prologue (W2 included) has landed before the loop:
  // the loop's own waits then follow its steady state only
  wide_w2_ready<KS>(rank, lane, w);
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  lds_barrier();

  // Iteration c (LDS stage c & 1) runs chunk c's MFMAs and, interleaved with
  // them, chunk c - 1's epilogue (its accumulators and inputs are ready), so
  // that no vector instruction waits on a result of the instructions just
  // before it (a SIMD does not run them under the MFMAs).  ha receives chunk
  // c + 2's W1 rows, hb holds chunk c + 1's (stored into stage (c + 1) & 1
  // at the end); uf holds chunk c - 1's epilogue inputs and then receives
  // chunk c + 1's.  Chunks past the last re-load the last one (never stored
  // differently), so every trip issues the same loads.
  //
  // Work besides the MFMAs runs in 64 sub-slots: sub-slot j right after
  // MFMA j * 4 KS / 64 of the iteration (one per MFMA at rank 512).
  //   0        row indices of chunk c + 2 (LDS)    2   its W1 rows (loads)
  //   3-50     draft: chunk c - 1's record (wide_draft_slot)
  //   4-52     residual: its epilogue steps 0-48 (wide_resid_step)
  //   kUSlot   chunk c + 1's epilogue inputs (after the pieces that read
  //            the previous ones)
  //   60       chunk c + 1's W1 rows into LDS
  constexpr int kUSlot = RESID ? 4 + kEpiSteps : kDraftUFree;
  constexpr int kPerH = WideH<KS>::kPer, kG = WideH<KS>::kGroups;
  constexpr int kSubPerMfma = 64 / (4 * KS);
  f32x4_t acc0[4], acc1[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc1[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto iter = [&](int c, int s, WideH<KS>& ha, WideH<KS>& hb, WideU<RESID>& uf, f32x4_t(&acc)[4],
                  const f32x4_t(&acc_prev)[4]) {
    const int c2 = min(c + 2, n_chunks - 1), c1 = min(c + 1, n_chunks - 1);
    const WideReq<RESID>* win2 = win[(c2 / kWideWinChunks) & 1] + (c2 % kWideWinChunks) * kWideChunk;
    const WideReq<RESID>* win1 = win[(c1 / kWideWinChunks) & 1];
    const uint16_t* w1 = static_cast<const uint16_t*>(p.W1);
    int hp[kPerH];
    WideEpi ep;
    WideDraftEpi dp;
    auto side = [&](int j) {
      if (j == 0) {
#pragma unroll
        for (int q = 0; q < kPerH; ++q) hp[q] = win2[min((tid + q * 256) / kG, kWideChunk - 1)].prev;
      } else if (j == 2) {
#pragma unroll
        for (int q = 0; q < kPerH; ++q) {
          const int g = (tid + q * 256) % kG;
          ha.v[q] = *reinterpret_cast<const u32x4_t*>(w1 + static_cast<int64_t>(hp[q]) * rank + min(g * 8, rank - 8));
        }
      }
      if constexpr (RESID) {
        if (j >= 4 && j < 4 + kEpiSteps) wide_resid_step(j - 4, p, seg, full, lane, uf, acc_prev, c > 0, ep);
      } else {
        if (j < kDraftEpiEnd) wide_draft_slot(j, p, seg, full, lane, uf, acc_prev, c > 0, dp);
      }
      if (j == kUSlot) wide_u_issue<RESID, VEC4>(p, win1, c1, c1 % kWideWinChunks, vw, lane, uf);
      if (j == 60) wide_h_commit<KS>(hb, rank, Hs + (s ^ 1) * kStage);
    };
    const uint16_t* hbase = Hs + s * kStage + (lane & 15) * RS + (lane >> 4) * 8;
    u32x4_t bq = *reinterpret_cast<const u32x4_t*>(hbase);
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t bn = bq;
      if (ks + 1 < KS) bn = *reinterpret_cast<const u32x4_t*>(hbase + (ks + 1) * 32);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w[b][ks]),
                                                         __builtin_bit_cast(bf16x8_t, bq), acc[b], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < kSubPerMfma; ++t) side((4 * ks + b) * kSubPerMfma + t);
        // nothing moves across: each sub-slot's work issues behind its MFMA
        __builtin_amdgcn_sched_barrier(0);
      }
      bq = bn;
    }
    // window wn + 1 is loaded at the window's first chunk and stored at its
    // ninth (its previous occupant, window wn - 1, is no longer read)
    const int wn = c / kWideWinChunks, cw = c % kWideWinChunks;
    if (wn + 1 < n_win) {
      if (cw == 0) wide_raw_load<RESID>(p, (wn + 1) * kWideWin + tid, cnt, raw);
      if (cw == kWideWinChunks / 2)
        wide_raw_store<RESID>(p, (wn + 1) * kWideWin + tid, cnt, raw, win[(wn + 1) & 1][tid]);
    }
    lds_barrier();
  };
  // whole pairs only (a loop exit between the two halves would give the
  // compiler a path that skips the second half's loads, and every wait in
  // the loop would be computed for it); with an odd count the last trip's
  // second half recomputes the last chunk, storing the same records again
  int c = 0;
  do {
    iter(c, 0, h0, h1, ua, acc0, acc1);
    iter(c + 1, 1, h1, h0, ub, acc1, acc0);
    c += 2;
  } while (c < n_chunks);
  // the last trip's second chunk
  if constexpr (RESID) {
    WideEpi ep;
#pragma unroll
    for (int t = 0; t < kEpiSteps; ++t) wide_resid_step(t, p, seg, full, lane, ua, acc1, true, ep);
  } else {
    WideDraftEpi dp;
#pragma unroll
    for (int j = 0; j < kDraftEpiEnd; ++j) wide_draft_slot(j, p, seg, full, lane, ua, acc1, true, dp);
  }
}

// ---------------------------------------------------------------------------
// 32-row path (fp32 weights): one wavefront = one 32-row segment, requests
// in chunks of 32
// ---------------------------------------------------------------------------
__device__ __forceinline__ int acc32_row(int i, int khalf) { return 8 * (i >> 2) + 4 * khalf + (i & 3); }

// Loads this lane's 16 logits of one request row for the 32x32 layout.
template <bool VEC4>
__device__ __forceinline__ void load16_32(const float* row, int vbase, int V, float (&x)[16]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4_t t = load4<VEC4>(row, vbase + 8 * g, V);
    x[4 * g + 0] = t[0];
    x[4 * g + 1] = t[1];
    x[4 * g + 2] = t[2];
    x[4 * g + 3] = t[3];
  }
}

// Per-wave record of one 32-row segment for the lane's request.
template <bool RESID, bool VEC4>
__device__ __forceinline__ void seg32_epilogue(const TileParams& p, const ReqInfo& ci, bool okn, int n, int seg,
                                               int khalf, const f32x16_t& acc, const float (&x)[16]) {
  const int V = p.V;
  const int vw = seg * kSegLarge;
  float rx, ry;
  if (!RESID) {
    float s[16];
    float m = -INFINITY;
    int im = kIntMax;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = vw + acc32_row(i, khalf);
      s[i] = (okn && v < V) ? acc[i] + x[i] : -INFINITY;
      const bool gt = s[i] > m;
      m = gt ? s[i] : m;
      im = gt ? v : im;
    }
    half_amax(m, im);
    // computed for greedy requests too (c = 0 gives 1s), then discarded
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) e += exp2_rel(s[i], m, ci.c);
    e = half_sum(e);
    rx = m;
    ry = (ci.c > 0.f) ? e : __int_as_float(im);
  } else {
    float t[16];
    load16_32<VEC4>(p.target + static_cast<int64_t>(ci.trow) * V, vw + 4 * khalf, V, t);
    float w = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = vw + acc32_row(i, khalf);
      const float q = exp2_hw((acc[i] + x[i] - ci.Mq) * ci.c) * ci.iZq;
      const float pp = exp2_hw((t[i] - ci.Mp) * ci.c) * ci.iZp;
      // masked rows add +0 (a bit mask, not a branch around the exps)
      const float d = fmaxf(pp - q, 0.f);
      w += __int_as_float(__float_as_int(d) & -static_cast<int>(okn && v < V));
    }
    w = half_sum(w);
    rx = 0.f;
    ry = w;
  }
  if (khalf == 0 && okn) {
    float2* rec = reinterpret_cast<float2*>(p.part) + static_cast<int64_t>(n) * p.n_seg + seg;
    *rec = make_float2(rx, ry);
  }
}

template <bool RESID, bool VEC4>
__global__ void __launch_bounds__(256) bias_seg32_f32(TileParams p) {
  constexpr int NCH = 32;
  constexpr int RS = DSPARK_MAX_RANK + 4;
  __shared__ __attribute__((aligned(16))) float Hf[NCH * RS];
  __shared__ ReqInfo s_ci[NCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, khalf = lane >> 5;
  const int seg = blockIdx.x * 4 + wave;
  const int V = p.V, rank = p.rank, R = p.R;

  if (RESID) {
    int any = 0;
    for (int n = tid; n < R; n += 256) any |= p.rs_info[4 * static_cast<int64_t>(n)];
    if (!__syncthreads_or(any)) return;
  }
  const int v_a = seg * kSegLarge + lrow;
  const float* w2row = static_cast<const float*>(p.W2) + static_cast<int64_t>(min(v_a, V - 1)) * rank;
  for (int n0 = 0; n0 < R; n0 += NCH) {
    lds_barrier();
    if (tid < NCH) s_ci[tid] = fetch_info(p, pos_of(p), n0 + tid, RESID);
    lds_barrier();
    {
      const float* w1 = static_cast<const float*>(p.W1);
      for (int q = tid; q < NCH * rank; q += 256) {
        const int nn = q / rank, k = q - nn * rank;
        const ReqInfo& ci = s_ci[nn];
        Hf[nn * RS + k] = ci.act ? w1[static_cast<int64_t>(ci.prev) * rank + k] : 0.0f;
      }
    }
    float x[16];
    {
      const int n = n0 + lrow;
      load16_32<VEC4>(u_row(p, pos_of(p), s_ci[lrow], n < R ? n : 0, RESID), seg * kSegLarge + 4 * khalf, V, x);
    }
    lds_barrier();
    f32x16_t acc = f32x16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* hrow = &Hf[lrow * RS + khalf];
    for (int ks = 0; ks < rank / 2; ++ks) {
      const float a = (v_a < V) ? w2row[2 * ks + khalf] : 0.0f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, hrow[2 * ks], acc, 0, 0, 0);
    }
    if (seg < p.n_seg) {
      const int n = n0 + lrow;
      const ReqInfo& ci = s_ci[lrow];
      seg32_epilogue<RESID, VEC4>(p, ci, (n < R) && ci.act, n, seg, khalf, acc, x);
    }
  }
}

// One launch, with the optional timing events attached to the dispatch.
template <typename K>
void launch(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const TileParams& p) {
  if (ev0 != nullptr || ev1 != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev0, ev1, 0, p);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, p);
}

// KS = seg16_ksteps(rank): the packed W2 layout uses the same count
template <bool RESID, bool VEC4, bool PACKED, int NB, bool SPLIT>
void launch_seg16_nb(const TileParams& p, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (seg16_ksteps(p.rank)) {
    case 2:
      if (RESID) launch(bias_seg16_res<2, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      else launch(bias_seg16<2, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      break;
    case 4:
      if (RESID) launch(bias_seg16_res<4, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      else launch(bias_seg16<4, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      break;
    case 8:
      if (RESID) launch(bias_seg16_res<8, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      else launch(bias_seg16<8, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      break;
    default:
      if (RESID) launch(bias_seg16_res<16, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      else launch(bias_seg16<16, VEC4, PACKED, NB, SPLIT>, grid, block, s, e0, e1, p);
      break;
  }
}

// request column blocks: as many as the batch needs (1, 2 or 4); H from
// W1[prev] (Markov head) or split from the fp32 states (RNN head)
template <bool RESID, bool VEC4, bool PACKED, bool SPLIT>
void launch_seg16_h(const TileParams& p, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.R <= 16)
    launch_seg16_nb<RESID, VEC4, PACKED, 1, SPLIT>(p, grid, block, s, e0, e1);
  else if (p.R <= 32)
    launch_seg16_nb<RESID, VEC4, PACKED, 2, SPLIT>(p, grid, block, s, e0, e1);
  else
    launch_seg16_nb<RESID, VEC4, PACKED, 4, SPLIT>(p, grid, block, s, e0, e1);
}

template <bool RESID, bool VEC4, bool PACKED>
void launch_seg16(const TileParams& p, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.h_base != nullptr)
    launch_seg16_h<RESID, VEC4, PACKED, true>(p, grid, block, s, e0, e1);
  else
    launch_seg16_h<RESID, VEC4, PACKED, false>(p, grid, block, s, e0, e1);
}

template <bool RESID, bool VEC4>
hipError_t launch_mode(const TileParams& p, int wdtype, int num_cu, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (wdtype == DSPARK_W_F32) {
    launch(bias_seg32_f32<RESID, VEC4>, dim3((p.n_seg + 3) / 4), dim3(256), s, e0, e1, p);
    return hipGetLastError();
  }
  if (p.seg_rows == kSegSmall) {
    // persistent: one workgroup per CU (draft: eight wavefronts, residual: four)
    const int wpb = RESID ? kSeg16Waves : kSeg16DraftWaves;
    // as many rounds of segments as one workgroup per CU needs, spread
    // evenly: every wavefront gets the same count, or one fewer
    const int n_walk = p.n_seg + p.n_seg_a;  // with the RNN head's A segments (draft mode)
    const int rounds = max(1, (n_walk + wpb * num_cu - 1) / (wpb * num_cu));
    const int blocks = max(1, min((n_walk + wpb * rounds - 1) / (wpb * rounds), num_cu));
    const dim3 grid(blocks), block(wpb * 64);
    if (p.w2p != nullptr)
      launch_seg16<RESID, VEC4, true>(p, grid, block, s, e0, e1);
    else
      launch_seg16<RESID, VEC4, false>(p, grid, block, s, e0, e1);
    return hipGetLastError();
  }
  // 64-row path: one workgroup per 256 vocabulary rows
  const dim3 grid((p.n_seg + 3) / 4), block(256);
  if (p.rank <= 64)
    launch(bias_seg64<2, RESID, VEC4>, grid, block, s, e0, e1, p);
  else if (p.rank <= 128)
    launch(bias_seg64<4, RESID, VEC4>, grid, block, s, e0, e1, p);
  else if (p.rank <= 256)
    launch(bias_seg64<8, RESID, VEC4>, grid, block, s, e0, e1, p);
  else
    launch(bias_seg64<16, RESID, VEC4>, grid, block, s, e0, e1, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bias_tile(const TileParams& p, int wdtype, bool residual, int num_cu, hipStream_t s,
                            hipEvent_t ev0, hipEvent_t ev1) {
  if (p.R == 0 || p.n_seg == 0) return hipSuccess;
  if (residual && (p.u_rows < 1 || p.t_rows < 1)) return hipErrorInvalidValue;
  // the 16-row path holds at most kSmallMaxR requests (LDS tile, record rows)
  if (p.seg_rows == kSegSmall && (p.R > kSmallMaxR || wdtype != DSPARK_W_BF16)) return hipErrorInvalidValue;
  // the 64-row path: bf16 weights; residual mode walks the verify list
  if (p.seg_rows == kSegWide &&
      (wdtype != DSPARK_W_BF16 || (residual && (p.rs_count == nullptr || p.rs_list == nullptr))))
    return hipErrorInvalidValue;
  // 32-row segments are the fp32-weight path only
  if (p.seg_rows == kSegLarge && wdtype != DSPARK_W_F32) return hipErrorInvalidValue;
  // H from the RNN head's states: the 16-row path only; A segments in its
  // draft mode only, with A (and with the packed W2, A's packed copy)
  if (p.h_base != nullptr && p.seg_rows != kSegSmall) return hipErrorInvalidValue;
  if (p.n_seg_a != 0 && (residual || p.h_base == nullptr || p.A == nullptr || p.z_out == nullptr ||
                         (p.w2p != nullptr && p.ap == nullptr) || p.n_seg_a < 0 ||
                         p.n_seg_a > (p.rank + kSegSmall - 1) / kSegSmall))
    return hipErrorInvalidValue;
  const bool vec4 = (p.V % 4) == 0;
  if (residual)
    return vec4 ? launch_mode<true, true>(p, wdtype, num_cu, s, ev0, ev1)
                : launch_mode<true, false>(p, wdtype, num_cu, s, ev0, ev1);
  return vec4 ? launch_mode<false, true>(p, wdtype, num_cu, s, ev0, ev1)
              : launch_mode<false, false>(p, wdtype, num_cu, s, ev0, ev1);
}

}  // namespace dspark
