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
#include "launchers.h"
#include "plan.h"
#include "sample_device.h"

namespace dspark {
namespace {

// Rescan of one record segment: thread group i (NT / seg_rows lanes) owns
// row v0 + i (256 threads: 16 lanes per row for 16-row segments, 8 for
// 32-row, 4 for 64-row; 1024 threads: four times as many).
template <int NT = 256>
__device__ __forceinline__ int lanes_log2(int seg_rows) {
  constexpr int extra = NT == 1024 ? 2 : 0;
  return (seg_rows == kSegSmall ? 4 : (seg_rows == kSegLarge ? 3 : 2)) + extra;
}
constexpr int kMaxSegRows = 64;
// threads per workgroup of the draft finish (bf16 weights, at most one
// request per CU): its per-thread share of the record pass (n_seg / NT
// records, read one after another) sets the location's latency
constexpr int kDraftFinishThreads = 1024;

// Segment records of one request staged in LDS: up to 2048 records (16 KiB,
// several workgroups per CU) or 16384 (128 KiB, i.e. V up to 262144 with
// 16-row, 524288 with 32-row or 1048576 with 64-row segments); larger
// vocabularies read the records from global memory instead.
constexpr int kStageSmall = 2048;
constexpr int kStageRecs = 16384;
constexpr int kStageBatchRecs = 10240;  // records in flight per workgroup while staging

// Records are copied into LDS in batches of kStageBatchRecs (kStageBatchRecs
// / NT loads per thread), every load of a batch issued before any is used
// (one memory latency per batch).
template <int NT = 256>
struct StageBatch {
  static constexpr int kLoads = kStageBatchRecs / NT;
  float2 r[kLoads];
};

template <int NT = 256>
__device__ __forceinline__ void stage_issue(const float2* __restrict__ src, int n, int base, StageBatch<NT>& b) {
#pragma unroll
  for (int j = 0; j < StageBatch<NT>::kLoads; ++j)
    b.r[j] = src[min(base + j * NT + static_cast<int>(threadIdx.x), n - 1)];
}

// Stores a batch into LDS, folding each record into f(r).  No barrier.
template <int NT = 256, class F>
__device__ __forceinline__ void stage_commit(int n, int base, const StageBatch<NT>& b, float2* dst, F f) {
#pragma unroll
  for (int j = 0; j < StageBatch<NT>::kLoads; ++j) {
    const int t = base + j * NT + static_cast<int>(threadIdx.x);
    if (t < n) {
      dst[t] = b.r[j];
      f(b.r[j]);
    }
  }
}

// h = W1[prev, :] as fp32, split so that its loads can be in flight with
// the record loads: hold() issues them into registers, commit() stores to
// LDS (no barrier).
template <typename WT, int NT = 256>
struct HRow {
  static constexpr int kPer = (DSPARK_MAX_RANK + NT - 1) / NT;
  float v[kPer];
  __device__ __forceinline__ void hold(const WT* W1, int prev, int rank) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = static_cast<int>(threadIdx.x) + j * NT;
      v[j] = weight_at<WT>(W1, static_cast<int64_t>(prev) * rank + min(k, rank - 1));
    }
  }
  __device__ __forceinline__ void commit(int rank, float* hs) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = static_cast<int>(threadIdx.x) + j * NT;
      if (k < rank) hs[k] = v[j];
    }
  }
};

// Block-wide (max, lowest index) with one barrier; lm / li are used once.
template <int NT = 256>
__device__ __forceinline__ void block_amax_once(float& m, int& i, float* lm, int* li) {
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
  for (int w = 1; w < NT / 64; ++w) amax_merge(m, i, lm[w], li[w]);
}

template <typename WT, int STAGE, int NT>
__global__ void __launch_bounds__(NT) draft_finish_kernel(FinishParams p) {
  constexpr bool STAGED = STAGE > 0;
  __shared__ float hs[DSPARK_MAX_RANK];
  __shared__ Loc2Scratch sh;
  __shared__ float e64[kMaxSegRows], s64[kMaxSegRows];
  __shared__ float2 srec[STAGED ? STAGE : 1];
  const int n = blockIdx.x, tid = threadIdx.x;
  const int V = p.V, n_seg = p.n_seg;
  if (p.err_clear != nullptr && (n | tid) == 0) *p.err_clear = 0u;
  const float2* gfine = reinterpret_cast<const float2*>(p.part) + static_cast<int64_t>(n) * n_seg;
  const float2* fine = STAGED ? srec : gfine;
  const int64_t o = static_cast<int64_t>(n) * p.gamma + p.k;
  // loads that depend on nothing go first; then the records, then W1[prev]
  // (whose address waits only for prev), all in flight together
  const float T = p.temp[n];
  const int prev = clampi(p.prev_base[static_cast<int64_t>(n) * p.prev_stride], 0, V - 1);
  const float u_raw = p.u_draft[o];
  StageBatch<NT> sb;
  if (STAGED) stage_issue<NT>(gfine, n_seg, 0, sb);
  HRow<WT, NT> hrow;
  hrow.hold(static_cast<const WT*>(p.W1), prev, p.rank);
  // maximum (greedy: with the lowest argmax carried in the records' second
  // word; sampled: the second word is ignored), taken while staging
  float m = -INFINITY;
  int im = kIntMax;
  auto fold = [&](float2 r) { amax_merge(m, im, r.x, __float_as_int(r.y)); };
  if (STAGED) {
    stage_commit<NT>(n_seg, 0, sb, srec, fold);
    for (int base = kStageBatchRecs; base < n_seg; base += kStageBatchRecs) {
      stage_issue<NT>(gfine, n_seg, base, sb);
      stage_commit<NT>(n_seg, base, sb, srec, fold);
    }
  } else {
#pragma unroll 8
    for (int t = tid; t < n_seg; t += NT) fold(gfine[t]);
  }
  hrow.commit(p.rank, hs);
  block_amax_once<NT>(m, im, sh.fred, sh.ired);  // also orders the LDS stores above before the reads below
  const float M = m;
  const float c = temp_scale(T);
  if (c == 0.0f) {
    if (tid == 0) {
      p.y[o] = clampi(im, 0, V - 1);
      p.q_tok[o] = 1.0f;
      p.q_stats[2 * o] = M;
      p.q_stats[2 * o + 1] = 1.0f;
    }
    return;
  }
  const float u = clamp_uniform(u_raw);
  // mass of segment t in units of 2^((. - M) c)
  auto mass = [&](int t) {
    const float2 r = fine[t];
    return r.y * exp2_hw((r.x - M) * c);
  };
  const Located2 L = locate_blocked<NT>(n_seg, mass, u, &sh);
  const int seg = L.seg < 0 ? 0 : L.seg;
  const float ms = fine[seg].x;
  const float th = L.fallback ? INFINITY : L.rem / exp2_hw((ms - M) * c);
  const int lg = lanes_log2<NT>(p.seg_rows);
  const int v0 = seg * p.seg_rows;
  const int i = tid >> lg;
  const int v = v0 + i;
  // the row's base logit is loaded before the W2 row, so both are in flight
  // together (clamped address; rows past V are masked below)
  const float uv = p.U_base[static_cast<int64_t>(n) * p.U_stride + min(v, V - 1)];
  const float b = row_bias<WT>(static_cast<const WT*>(p.W2), hs, p.rank, v, V, lg);
  if ((tid & ((1 << lg) - 1)) == 0) {
    float s = -INFINITY, e = 0.0f;
    if (v < V) {
      s = uv + b;
      e = exp2_hw((s - ms) * c);
    }
    e64[i] = e;
    s64[i] = s;
  }
  __syncthreads();
  if (tid < 64) {
    const int pos = pick64(e64, p.seg_rows, th);
    if (tid == 0) {
      const int yy = (pos >= 0) ? v0 + pos : min(v0, V - 1);
      const float sy = (pos >= 0) ? s64[pos] : M;
      p.y[o] = yy;
      p.q_tok[o] = exp2_hw((sy - M) * c) / L.Z;
      p.q_stats[2 * o] = M;
      p.q_stats[2 * o + 1] = L.Z;
    }
  }
}

template <typename WT, int STAGE>
__global__ void __launch_bounds__(256) residual_finish_kernel(VerifyParams p) {
  constexpr bool STAGED = STAGE > 0;
  __shared__ float hs[DSPARK_MAX_RANK];
  __shared__ Loc2Scratch sh2;
  __shared__ ChunkScratch sh;
  __shared__ float e64[kMaxSegRows];
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
      float w = 0.0f;
      if (v < V) {
        const float s = uv + b;
        const float q = exp2_hw((s - Mq) * c) * iZq;
        const float pp = exp2_hw((tv - Mp) * c) * iZp;
        w = fmaxf(pp - q, 0.0f);
      }
      e64[i] = w;
    }
    __syncthreads();
    if (tid < 64) {
      const int pos = pick64(e64, p.seg_rows, th);
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
  else if (stage == kStageRecs)
    hipLaunchKernelGGL((draft_finish_kernel<WT, kStageRecs, NT>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((draft_finish_kernel<WT, 0, NT>), grid, block, 0, s, p);
}

hipError_t launch_draft_finish(const FinishParams& p, int wdtype, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const int num_cu = current_cu_count();
  const int stage = p.n_seg <= kStageSmall ? kStageSmall : (p.n_seg <= kStageRecs ? kStageRecs : 0);
  // 1024 threads while every request's workgroup gets a CU of its own; more
  // requests than CUs run as several smaller workgroups per CU instead.  fp32
  // weights: the 32-row rescan's registers fit 256 threads per workgroup.
  if (wdtype == DSPARK_W_BF16 && p.R <= num_cu)
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
  const int stage = p.n_seg <= kStageSmall ? kStageSmall : (p.n_seg <= kStageRecs ? kStageRecs : 0);
  if (wdtype == DSPARK_W_BF16) {
    if (stage == kStageSmall)
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, kStageSmall>), grid, block, 0, s, p);
    else if (stage == kStageRecs)
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, kStageRecs>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((residual_finish_kernel<uint16_t, 0>), grid, block, 0, s, p);
  } else {
    if (stage == kStageSmall)
      hipLaunchKernelGGL((residual_finish_kernel<float, kStageSmall>), grid, block, 0, s, p);
    else if (stage == kStageRecs)
      hipLaunchKernelGGL((residual_finish_kernel<float, kStageRecs>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((residual_finish_kernel<float, 0>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace dspark
