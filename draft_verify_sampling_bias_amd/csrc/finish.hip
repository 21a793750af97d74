// Per-request finish kernels of the draft and of the residual correction.
//
// Draft (one workgroup per request, once per block position): combines the
// segment records of the fused bias kernel into the position's maximum,
// lowest argmax and normaliser Z, and for a sampled request draws the token by
// inverse CDF with its uniform ("DSpark" explainer sections 2 and 7: the
// block is drafted left to right from q = softmax((U_k + B_k)/T); llama.cpp
// PR #25173: anchor-first, bias(prev) = markov_w2 . markov_w1[prev]).
//
// Residual (one workgroup per request that rejected a sampled draft): draws
// the correction from max(0, p - q) normalised (explainer section 3), using
// the segment sums written by the residual pass of the fused bias kernel; if
// that residual has no mass it draws from p.


#include "device_info.h"
#include "dspark_device.h"
#include "finish_device.h"
#include "launchers.h"
#include "plan.h"
#include "sample_device.h"

namespace dspark {
namespace {

// Relative distance within which the residual rescan's recomputed segment
// maximum counts as the draft's maximum (rounding of fp32 dot products of
// up to 512 terms in two summation orders stays far below it).
constexpr float kRoundSnap = 0x1p-16f;
// magnitude below which the distance is taken absolute (2^-16 * 2^-10): a
// maximum of exactly 0 still admits the rounding of its dot product
constexpr float kRoundFloor = 0x1p-10f;

template <typename WT, int STAGE, int NT>
__global__ void __launch_bounds__(NT) draft_finish_kernel(FinishParams p) {
  __shared__ FinishSmem sm;
  __shared__ float2 srec[STAGE > 0 ? STAGE : 1];
  if (p.err_clear != nullptr && (blockIdx.x | threadIdx.x) == 0) *p.err_clear = 0u;
  draft_finish_one<WT, STAGE, NT>(p, blockIdx.x, p.k, p.prev_base, p.prev_stride, p.U_base, sm, srec);
}

template <typename WT, int NT, int J, int SEG>
__global__ void __launch_bounds__(NT) draft_finish_waves_kernel(FinishParams p) {
  __shared__ WaveFinishSmem<NT> sm;
  if (p.err_clear != nullptr && (blockIdx.x | threadIdx.x) == 0) *p.err_clear = 0u;
  draft_finish_waves<WT, NT, J, SEG>(p, sm);
}

// the wave-range finish with records per lane J chosen from n_seg
template <int NT, int SEG>
void launch_draft_finish_waves(const FinishParams& p, hipStream_t s) {
  const dim3 grid(p.R), block(NT);
  if (p.n_seg <= NT * 4)
    hipLaunchKernelGGL((draft_finish_waves_kernel<uint16_t, NT, 4, SEG>), grid, block, 0, s, p);
  else if (p.n_seg <= NT * 8)
    hipLaunchKernelGGL((draft_finish_waves_kernel<uint16_t, NT, 8, SEG>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((draft_finish_waves_kernel<uint16_t, NT, kWaveFinishJ, SEG>), grid, block, 0, s, p);
}

template <typename WT, int STAGE>
__global__ void __launch_bounds__(256) residual_finish_kernel(VerifyParams p) {
  constexpr bool STAGED = STAGE > 0;
  __shared__ float hs[DSPARK_MAX_RANK];
  __shared__ Loc2Scratch sh2;
  __shared__ ChunkScratch sh;
  __shared__ float s64[kMaxSegRows], t64[kMaxSegRows];
  __shared__ int s_out;
  __shared__ float2 srec[STAGED ? STAGE : 1];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int32_t* info = p.rs_info + 4 * static_cast<int64_t>(n);
  if (info[0] == 0) return;
  const int V = p.V;
  const int prev = clampi(info[1], 0, V - 1);
  const int64_t urow = min(max(static_cast<int64_t>(info[2]), int64_t{0}), static_cast<int64_t>(p.R) * p.gamma - 1);
  const int64_t trow = min(max(static_cast<int64_t>(info[3]), int64_t{0}), p.n_rows - 1);
  const float* st = p.rs_stats + 4 * static_cast<int64_t>(n);
  const float Mq = st[0], iZq = 1.0f / st[1], Mp = st[2], iZp = 1.0f / st[3];
  const float c = temp_scale(p.temp[n]);
  const float u = clamp_uniform(p.u_final[n]);
  const float2* gfine = reinterpret_cast<const float2*>(p.rpart) + static_cast<int64_t>(n) * p.n_seg;
  const float2* fine = STAGED ? srec : gfine;
  StageBatch<256> sb;
  if (STAGED) stage_issue<256>(gfine, p.n_seg, 0, sb);
  HRow<WT, 256> hrow;
  if (p.hstate != nullptr)
    hrow.hold_state(p.hstate + urow * p.rank, p.rank);
  else
    hrow.hold(static_cast<const WT*>(p.W1), prev, p.rank);
  if (STAGED) {
    auto none = [](float2) {};
    stage_commit<256>(p.n_seg, 0, sb, srec, none);
    for (int base = kStageBatchRecs; base < p.n_seg; base += kStageBatchRecs) {
      stage_issue<256>(gfine, p.n_seg, base, sb);
      stage_commit<256>(p.n_seg, base, sb, srec, none);
    }
  }
  hrow.commit(p.rank, hs);
  __syncthreads();
  auto mass = [&](int t) { return fine[t].y; };
  const Located2 L = locate_blocked(p.n_seg, mass, u, &sh2);
  const float* tr = p.target + trow * V;
  int out = -1;
  if (L.Z > 0.0f && L.seg >= 0) {
    const float th = L.fallback ? INFINITY : L.rem;
    const int lg = lanes_log2<256>(p.seg_rows);
    const int v0 = L.seg * p.seg_rows;
    const int i = tid >> lg;
    const int v = v0 + i;
    // the row's base and target logits are loaded before the W2 row, so all
    // are in flight together (clamped addresses; rows past V are masked below)
    const int vc = min(v, V - 1);
    const float uv = p.U[urow * V + vc], tv = tr[vc];
    const float b = row_bias<WT>(static_cast<const WT*>(p.W2), hs, p.rank, v, V, lg);
    if ((tid & ((1 << lg) - 1)) == 0) {
      s64[i] = (v < V) ? uv + b : -INFINITY;
      t64[i] = (v < V) ? tv : -INFINITY;
    }
    __syncthreads();
    if (tid < 64) {
      const int ns = p.seg_rows;
      const float sv = tid < ns ? s64[tid] : -INFINITY, tl = tid < ns ? t64[tid] : -INFINITY;
      // q relative to the draft's maximum Mq.  The rescanned logits can
      // differ from the records' by rounding (fp32 weights summed in another
      // order than the fused kernel's, which gave the top row exactly Mq);
      // when the segment's own maximum lies within that rounding of Mq and
      // c would still magnify the difference beyond a factor of 2, the
      // segment holds the top row and its own maximum is the reference.
      float mr = sv;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) mr = fmaxf(mr, __shfl_xor(mr, d));
      const float dq = mr - Mq;
      const float ref = (fabsf(dq) <= kRoundSnap * fmaxf(fabsf(Mq), kRoundFloor) && fabsf(dq * c) > 1.0f) ? mr : Mq;
      const float q = (sv == -INFINITY) ? 0.0f : exp2_rel(sv, ref, c) * iZq;
      const float pp = exp2_hw((tl - Mp) * c) * iZp;
      const int pos = pick64_reg(tid < ns ? fmaxf(pp - q, 0.0f) : 0.0f, th);
      if (tid == 0) s_out = (pos >= 0) ? v0 + pos : -1;
    }
    __syncthreads();
    out = s_out;
  }
  if (out < 0) {
    // no residual mass: the correction is drawn from p itself
    out = chunk_draw(p.vpart + trow * p.n_chunks * kChunkFloats, p.n_chunks, tr, V, Mp, c, u, &sh);
  }
  if (tid == 0) p.out_tok[n] = clampi(out, 0, V - 1);
}

}  // namespace

template <typename WT, int NT>
void launch_draft_finish_nt(const FinishParams& p, int stage, hipStream_t s) {
  const dim3 grid(p.R), block(NT);
  if (stage == kStageSmall)
    hipLaunchKernelGGL((draft_finish_kernel<WT, kStageSmall, NT>), grid, block, 0, s, p);
  else if (stage == kStageMid)
    hipLaunchKernelGGL((draft_finish_kernel<WT, kStageMid, NT>), grid, block, 0, s, p);
  else if (stage == kStageMid2)
    hipLaunchKernelGGL((draft_finish_kernel<WT, kStageMid2, NT>), grid, block, 0, s, p);
  else if (stage == kStageRecs)
    hipLaunchKernelGGL((draft_finish_kernel<WT, kStageRecs, NT>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((draft_finish_kernel<WT, 0, NT>), grid, block, 0, s, p);
}

bool draft_finish_fuses_state(const FinishParams& p, int wdtype) {
  return wdtype == DSPARK_W_BF16 && p.seg_rows == kSegSmall && p.R <= current_cu_count() &&
         p.n_seg <= kDraftFinishThreads * kWaveFinishJ;
}

hipError_t launch_draft_finish(const FinishParams& p, int wdtype, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const int num_cu = current_cu_count();
  const int stage = stage_for(p.n_seg);
  // 1024 threads while every request's workgroup gets a CU of its own; more
  // requests than CUs run as several smaller workgroups per CU instead.  bf16
  // weights with 16- or 64-row segments take the wave-range finish (records
  // in registers) up to kWaveFinishJ records per lane, the staged-record
  // finish beyond.  fp32 weights: the 32-row rescan's registers fit 256
  // threads per workgroup.
  const bool waves = wdtype == DSPARK_W_BF16 && (p.seg_rows == kSegSmall || p.seg_rows == kSegWide);
  if (waves && p.R <= num_cu && p.n_seg <= kDraftFinishThreads * kWaveFinishJ) {
    if (p.seg_rows == kSegSmall)
      launch_draft_finish_waves<kDraftFinishThreads, kSegSmall>(p, s);
    else
      launch_draft_finish_waves<kDraftFinishThreads, kSegWide>(p, s);
  } else if (waves && p.seg_rows == kSegWide && p.n_seg <= 256 * kWaveFinishJ) {
    launch_draft_finish_waves<256, kSegWide>(p, s);
  } else if (wdtype == DSPARK_W_BF16 && p.R <= num_cu)
    launch_draft_finish_nt<uint16_t, kDraftFinishThreads>(p, stage, s);
  else if (wdtype == DSPARK_W_BF16)
    launch_draft_finish_nt<uint16_t, 256>(p, stage, s);
  else
    launch_draft_finish_nt<float, 256>(p, stage, s);
  return hipGetLastError();
}

hipError_t launch_residual_finish(const VerifyParams& p, int wdtype, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const dim3 grid(p.R), block(256);
  const int stage = stage_for(p.n_seg);
  if (wdtype == DSPARK_W_BF16) {
    if (stage == kStageSmall)
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, kStageSmall>), grid, block, 0, s, p);
    else if (stage == kStageMid)
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, kStageMid>), grid, block, 0, s, p);
    else if (stage == kStageMid2)
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, kStageMid2>), grid, block, 0, s, p);
    else if (stage == kStageRecs)
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, kStageRecs>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, 0>), grid, block, 0, s, p);
  } else {
    if (stage == kStageSmall)
      hipLaunchKernelGGL((residual_finish_kernel<float, kStageSmall>), grid, block, 0, s, p);
    else if (stage == kStageMid)
      hipLaunchKernelGGL((residual_finish_kernel<float, kStageMid>), grid, block, 0, s, p);
    else if (stage == kStageMid2)
      hipLaunchKernelGGL((residual_finish_kernel<float, kStageMid2>), grid, block, 0, s, p);
    else if (stage == kStageRecs)
      hipLaunchKernelGGL((residual_finish_kernel<float, kStageRecs>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((residual_finish_kernel<float, 0>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace dspark
