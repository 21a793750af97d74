// Device code of the per-request draft finish (finish.hip), written as one
// request's finish by one workgroup so that any kernel can run it.
//
// The finish combines the segment records of the fused bias kernel into the
// position's maximum, lowest argmax and normaliser Z, and for a sampled
// request draws the token by inverse CDF with its uniform ("DSpark"
// explainer sections 2 and 7: the block is drafted left to right from
// q = softmax((U_k + B_k)/T); llama.cpp PR #25173: anchor-first,
// bias(prev) = markov_w2 . markov_w1[prev]).
#pragma once

#include "dspark_device.h"
#include "launchers.h"
#include "plan.h"
#include "sample_device.h"

namespace dspark {

// Rescan of one record segment: thread group i (NT / seg_rows lanes) owns
// row v0 + i (256 threads: 16 lanes per row for 16-row segments, 8 for
// 32-row; 512 and 1024 threads: two and four times as many).
template <int NT = 256>
__device__ __forceinline__ int lanes_log2(int seg_rows) {
  static_assert(NT == 256 || NT == 512 || NT == 1024, "finish workgroups of 256, 512 or 1024 threads");
  constexpr int extra = NT == 1024 ? 2 : (NT == 512 ? 1 : 0);
  return (seg_rows == kSegSmall ? 4 : (seg_rows == kSegLarge ? 3 : 2)) + extra;
}
constexpr int kMaxSegRows = 64;
// threads per workgroup of the draft finish (bf16 weights, at most one
// request per CU): its per-thread share of the record pass (n_seg / NT
// records, read one after another) sets the location's latency
constexpr int kDraftFinishThreads = 1024;

// Segment records of one request staged in LDS: up to 2048, 4096 or 8192
// records (16, 32 or 64 KiB: several workgroups per CU) or 16384 (128 KiB,
// i.e. V up to 262144 with 16-row or 524288 with 32-row segments); larger
// vocabularies read the records from global memory instead.
constexpr int kStageSmall = 2048;
constexpr int kStageMid = 4096;
constexpr int kStageMid2 = 8192;
constexpr int kStageRecs = 16384;
// the smallest stage that holds n_seg records, or 0 (read from global memory)
inline int stage_for(int n_seg) {
  return n_seg <= kStageSmall ? kStageSmall
                              : (n_seg <= kStageMid ? kStageMid
                                                    : (n_seg <= kStageMid2 ? kStageMid2
                                                                           : (n_seg <= kStageRecs ? kStageRecs : 0)));
}
constexpr int kStageBatchRecs = 10240;  // records in flight per workgroup while staging

// Records are copied into LDS in batches of kStageBatchRecs (kStageBatchRecs
// / NT loads per thread), every load of a batch issued before any is used
// (one memory latency per batch).
template <int NT = 256, int BATCH = kStageBatchRecs>
struct StageBatch {
  static constexpr int kLoads = BATCH / NT;
  float2 r[kLoads];
};

template <int NT = 256, int BATCH = kStageBatchRecs>
__device__ __forceinline__ void stage_issue(const float2* __restrict__ src, int n, int base,
                                            StageBatch<NT, BATCH>& b) {
#pragma unroll
  for (int j = 0; j < StageBatch<NT, BATCH>::kLoads; ++j)
    b.r[j] = src[min(base + j * NT + static_cast<int>(threadIdx.x), n - 1)];
}

// Stores a batch into LDS, folding each record into f(r).  No barrier.
template <int NT = 256, int BATCH = kStageBatchRecs, class F>
__device__ __forceinline__ void stage_commit(int n, int base, const StageBatch<NT, BATCH>& b, float2* dst, F f) {
#pragma unroll
  for (int j = 0; j < StageBatch<NT, BATCH>::kLoads; ++j) {
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
  // the RNN head's fp32 state row instead
  __device__ __forceinline__ void hold_state(const float* h, int rank) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int k = static_cast<int>(threadIdx.x) + j * NT;
      v[j] = h[min(k, rank - 1)];
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

// LDS of one draft finish, besides the record staging buffer.
struct FinishSmem {
  float hs[DSPARK_MAX_RANK];
  Loc2Scratch sh;
  float s64[kMaxSegRows];
};

// The draft finish of request n at position p.k, by one workgroup of NT
// threads: the position's maximum, lowest argmax and normaliser Z from the
// segment records, and for a sampled request the inverse-CDF draw of its
// uniform (two levels over the records, then a rescan of the chosen
// segment).  Writes y, q_tok and q_stats of (n, k).  The caller separates
// two calls on the same scratch with a workgroup barrier.
// SEG: the segment rows when known at compile time (0: p.seg_rows).
// Position k reads request n's previous token at prev_base[n * prev_stride]
// and its base logits at U_base + n * p.U_stride.  With STAGE > 0 the
// request's records (at most STAGE of them) are staged in srec (LDS), BATCH
// records in flight at a time.
template <typename WT, int STAGE, int NT, int SEG = 0, int BATCH = kStageBatchRecs>
__device__ __forceinline__ void draft_finish_one(const FinishParams& p, int n, int k, const int32_t* prev_base,
                                                 int prev_stride, const float* U_base, FinishSmem& sm,
                                                 float2* srec) {
  constexpr bool STAGED = STAGE > 0;
  float* hs = sm.hs;
  Loc2Scratch& sh = sm.sh;
  float* s64 = sm.s64;
  const int tid = threadIdx.x;
  const int V = p.V, n_seg = p.n_seg;
  const float2* gfine = reinterpret_cast<const float2*>(p.part) + static_cast<int64_t>(n) * n_seg;
  const float2* fine = STAGED ? srec : gfine;
  const int64_t o = static_cast<int64_t>(n) * p.gamma + k;
  // loads that depend on nothing go first; then the records, then W1[prev]
  // (whose address waits only for prev), all in flight together
  const float T = p.temp[n];
  const int prev = clampi(prev_base[static_cast<int64_t>(n) * prev_stride], 0, V - 1);
  const float u_raw = p.u_draft[o];
  StageBatch<NT, BATCH> sb;
  if (STAGED) stage_issue<NT, BATCH>(gfine, n_seg, 0, sb);
  HRow<WT, NT> hrow;
  if (p.hstate != nullptr)
    hrow.hold_state(p.hstate + o * p.rank, p.rank);
  else
    hrow.hold(static_cast<const WT*>(p.W1), prev, p.rank);
  // maximum (greedy: with the lowest argmax carried in the records' second
  // word; sampled: the second word is ignored), taken while staging
  float m = -INFINITY;
  int im = kIntMax;
  auto fold = [&](float2 r) { amax_merge(m, im, r.x, __float_as_int(r.y)); };
  if (STAGED) {
    stage_commit<NT, BATCH>(n_seg, 0, sb, srec, fold);
    for (int base = BATCH; base < n_seg; base += BATCH) {
      stage_issue<NT, BATCH>(gfine, n_seg, base, sb);
      stage_commit<NT, BATCH>(n_seg, base, sb, srec, fold);
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
  // the chosen segment's mass relative to its record maximum, and the
  // fraction of it left over by the search over the records
  const float rec = fine[seg].y;
  const float th = L.fallback ? INFINITY : L.rem / exp2_hw((ms - M) * c);
  const float frac = L.fallback ? INFINITY : (rec > 0.0f ? th / rec : 0.0f);
  const int seg_rows = SEG > 0 ? SEG : p.seg_rows;
  const int lg = lanes_log2<NT>(seg_rows);
  const int v0 = seg * seg_rows;
  const int i = tid >> lg;
  const int v = v0 + i;
  // the row's base logit is loaded before the W2 row, so both are in flight
  // together (clamped address; rows past V are masked below)
  const float uv = U_base[static_cast<int64_t>(n) * p.U_stride + min(v, V - 1)];
  // lanes per row known at compile time when SEG is: fewer weight chunks per lane
  constexpr int kMinLg = SEG > 0 ? (SEG == kSegSmall ? 4 : (SEG == kSegLarge ? 3 : 2)) + (NT == 1024 ? 2 : (NT == 512 ? 1 : 0)) : 2;
  const float b = row_bias<WT, kMinLg>(static_cast<const WT*>(p.W2), hs, p.rank, v, V, lg);
  if ((tid & ((1 << lg) - 1)) == 0) s64[i] = (v < V) ? uv + b : -INFINITY;
  __syncthreads();
  if (tid < 64) {
    // weights relative to the rescan's own maximum (seg_pick_own_max); q of
    // the drawn row = its share of the segment times the segment's share of Z
    const SegPick sp = seg_pick_own_max(tid < seg_rows ? s64[tid] : -INFINITY, seg_rows, c, frac);
    if (tid == 0) {
      const int yy = (sp.pos >= 0) ? v0 + sp.pos : min(v0, V - 1);
      p.y[o] = yy;
      p.q_tok[o] = (sp.pos >= 0) ? sp.qin * (rec * exp2_rel(ms, M, c) / L.Z) : 1.0f / L.Z;
      p.q_stats[2 * o] = M;
      p.q_stats[2 * o + 1] = L.Z;
    }
  }
}

// ---------------------------------------------------------------------------
// Wave-range draft finish (bf16 weights, 16- or 64-row segments, n_seg <=
// NT * kWaveFinishJ)
// ---------------------------------------------------------------------------
// Wavefront w owns the contiguous records [w P, w P + n_w) (P = ceil(n_seg /
// NW)); lane l holds records w P + 64 j + l (j < L = ceil(n_w / 64)) in
// registers, read with coalesced loads.  Each wavefront publishes one pair,
// (max, lowest argmax) for a greedy request or (max m_w, mass sum s_w in
// units of 2^((. - m_w) c)) for a sampled one, and the workgroup meets at
// its only barrier.  Every wavefront then combines the NW pairs, one per
// lane, in the same order, so all agree on M, Z and on the wavefront whose
// range holds u Z.  That wavefront alone finds the record: it transposes its
// masses through LDS so that lane l holds the run [l L, l L + L) of its
// range, scans the lanes' run sums and walks the chosen lane's run.  A
// 16-row segment it then rescans alone, four lanes per row; a 64-row one it
// hands to the whole workgroup through LDS (a second barrier), which
// rescans it with NT / 64 lanes per row before wavefront 0 picks the entry
// (a third).
constexpr int kWaveFinishJ = 12;  // records per lane at most (n_seg <= 12288 with 1024 threads)
template <int NT>
struct WaveFinishSmem {
  float hs[DSPARK_MAX_RANK];
  float wm[NT / 64];
  float ws[NT / 64];
  int wi[NT / 64];
  float tx[64 * kWaveFinishJ];  // the chosen wavefront's masses, then the chosen record (max, mass)
  // 64-row segments: the chosen segment, the fraction of its mass left over
  // by the search, its record's maximum and mass, and the rescanned rows'
  // logits
  int hseg;
  float hfrac, hms, hrec;
  float s64[kMaxSegRows];
  // RNN head, next state fused: the drafted token
  int ynext;
};

// The RNN head's next state, fused into the finish of (n, k < gamma - 1):
// the fused bias kernel has stored z = A h in the state row of (n, k + 1);
// this finish turns it into h = act(z + W1[y]), rounded to double-bf16 as
// the state kernel rounds it (thread j < rank holds z_j from its entry).
__device__ __forceinline__ void fused_state_store(const FinishParams& p, float zj, int y, int64_t o) {
  const int j = static_cast<int>(threadIdx.x);
  if (j < p.rank) {
    const uint16_t* w1 = static_cast<const uint16_t*>(p.W1) + static_cast<int64_t>(clampi(y, 0, p.V - 1)) * p.rank;
    p.hstate[(o + 1) * p.rank + j] = double_bf16(rnn_act(zj + bf16_to_f32(w1[j]), p.act));
  }
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// The chosen wavefront's second level (see draft_finish_waves) and, for a
// 16-row segment, its rescan and the stores; for a 64-row segment the
// hand-over of (segment, threshold, maximum) through LDS.
template <typename WT, int NT, int J, int SEG>
__device__ __forceinline__ void draft_finish_waves_pick(const FinishParams& p, WaveFinishSmem<NT>& sm,
                                                        const float2 (&r)[J], int n, int64_t o, int w0, int L,
                                                        float M, float Z, float c, float theta, float P, bool fb) {
  const int lane = threadIdx.x & 63;
  const int V = p.V;
  // second level: the masses of this wavefront's records (position q =
  // 64 j + lane of its range) through LDS to lane q / L, so that each lane
  // holds a run of consecutive records; the lane whose run holds th = theta
  // - P, then the first record of that run whose running mass passes it
  const float th = fb ? INFINITY : theta - P;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < L) sm.tx[j * 64 + lane] = r[j].y * exp2_rel(r[j].x, M, c);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int l0 = lane * L;
  float x[J];
  float tot = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    x[j] = (j < L) ? sm.tx[l0 + j] : 0.0f;
    tot += x[j];
  }
  const float cum = wave_incl_scan(tot);
  const float cup = __shfl_up(cum, 1);
  const float ex = (lane == 0) ? 0.0f : cup;
  // each lane walks its own run from its exclusive prefix: the first record
  // past th, and the last record with mass
  int jsel = -1, jlast = -1;
  float psel = 0.0f, plast = 0.0f, run = ex;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < L) {
      const float nxt = run + x[j];
      const bool pos = x[j] > 0.0f;
      const bool take = jsel < 0 && pos && nxt > th;
      psel = take ? run : psel;
      jsel = take ? j : jsel;
      plast = pos ? run : plast;
      jlast = pos ? j : jlast;
      run = nxt;
    }
  }
  const unsigned long long hit = __ballot(tot > 0.0f && cum > th);
  const unsigned long long any = __ballot(tot > 0.0f);
  int q = -1;  // position of the chosen record in the wavefront's range
  float selP = 0.0f;
  if (hit) {
    // the lane whose interval [ex, cum) holds th; if its own walk stops
    // short of th by rounding, its last record with mass is taken
    const int ls = __ffsll(static_cast<long long>(hit)) - 1;
    const int js = __builtin_amdgcn_readlane(jsel, ls);
    const bool found = js >= 0;
    q = ls * L + (found ? js : __builtin_amdgcn_readlane(jlast, ls));
    selP = readlane_f(found ? psel : plast, ls);
    fb = fb || !found;
  } else if (any) {
    const int ll = 63 - __clzll(static_cast<long long>(any));
    q = ll * L + __builtin_amdgcn_readlane(jlast, ll);
    selP = readlane_f(plast, ll);
    fb = true;
  } else {
    fb = true;
  }
  // the chosen record's maximum, through the same LDS (every lane has read
  // its masses above)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < L && j * 64 + lane == q) {
      sm.tx[0] = r[j].x;
      sm.tx[1] = r[j].y;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const float ms = q >= 0 ? sm.tx[0] : M;
  const float rec = q >= 0 ? sm.tx[1] : 0.0f;  // its mass relative to ms
  const int seg = q >= 0 ? w0 + q : 0;
  const float ths = fb ? INFINITY : (th - selP) / exp2_rel(ms, M, c);
  const float frac = fb ? INFINITY : (rec > 0.0f ? ths / rec : 0.0f);
  if constexpr (SEG == kSegWide) {
    if (lane == 0) {
      sm.hseg = seg;
      sm.hfrac = frac;
      sm.hms = ms;
      sm.hrec = rec;
    }
    return;
  }
  // rescan of the segment's 16 rows: four lanes per row
  const int v0 = seg * kSegSmall;
  const int i = lane >> 2;
  const int v = v0 + i;
  const float uv = p.U_base[static_cast<int64_t>(n) * p.U_stride + min(v, V - 1)];
  const float b = row_bias<WT, 2>(static_cast<const WT*>(p.W2), sm.hs, p.rank, v, V, 2);
  const float sv = (v < V) ? uv + b : -INFINITY;
  // row i's logit to lane i, then the pick in the segment with weights
  // relative to the rescan's own maximum (seg_pick_own_max)
  const float sl = __shfl(sv, (lane & 15) * 4);
  const SegPick sp = seg_pick_own_max(sl, kSegSmall, c, frac);
  if (lane == 0) {
    const int yy = (sp.pos >= 0) ? v0 + sp.pos : min(v0, V - 1);
    sm.ynext = yy;
    p.y[o] = yy;
    p.q_tok[o] = (sp.pos >= 0) ? sp.qin * (rec * exp2_rel(ms, M, c) / Z) : 1.0f / Z;
    p.q_stats[2 * o] = M;
    p.q_stats[2 * o + 1] = Z;
  }
}

// Rescan of the handed-over 64-row segment by the whole workgroup (NT / 64
// lanes per row), then wavefront 0's pick and the stores.
template <typename WT, int NT>
__device__ __forceinline__ void draft_finish_rescan64(const FinishParams& p, WaveFinishSmem<NT>& sm, int n, int64_t o,
                                                      float M, float Z, float c) {
  const int tid = threadIdx.x;
  const int V = p.V;
  const int seg = sm.hseg;
  const float frac = sm.hfrac, ms = sm.hms, rec = sm.hrec;
  constexpr int kLg = NT == 1024 ? 4 : (NT == 512 ? 3 : 2);  // log2 of the lanes per row
  const int v0 = seg * kSegWide;
  const int i = tid >> kLg;
  const int v = v0 + i;
  const float uv = p.U_base[static_cast<int64_t>(n) * p.U_stride + min(v, V - 1)];
  const float b = row_bias<WT, kLg>(static_cast<const WT*>(p.W2), sm.hs, p.rank, v, V, kLg);
  if ((tid & ((1 << kLg) - 1)) == 0) sm.s64[i] = (v < V) ? uv + b : -INFINITY;
  __syncthreads();
  if (tid < 64) {
    // weights relative to the rescan's own maximum (seg_pick_own_max)
    const SegPick sp = seg_pick_own_max(sm.s64[tid], kSegWide, c, frac);
    if (tid == 0) {
      const int yy = (sp.pos >= 0) ? v0 + sp.pos : min(v0, V - 1);
      p.y[o] = yy;
      p.q_tok[o] = (sp.pos >= 0) ? sp.qin * (rec * exp2_rel(ms, M, c) / Z) : 1.0f / Z;
      p.q_stats[2 * o] = M;
      p.q_stats[2 * o + 1] = Z;
    }
  }
}

template <typename WT, int NT, int J, int SEG>
__device__ __forceinline__ void draft_finish_waves(const FinishParams& p, WaveFinishSmem<NT>& sm) {
  static_assert(SEG == kSegSmall || SEG == kSegWide, "16- or 64-row segments");
  constexpr int NW = NT / 64;
  static_assert(NW <= 64, "one wavefront pair per lane");
  const int n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = p.V, n_seg = p.n_seg;
  const float2* rec = reinterpret_cast<const float2*>(p.part) + static_cast<int64_t>(n) * n_seg;
  const int64_t o = static_cast<int64_t>(n) * p.gamma + p.k;
  // loads that depend on nothing first, then the records, then h (whose
  // address waits only for prev), all in flight together
  const float T = p.temp[n];
  const int prev = clampi(p.prev_base[static_cast<int64_t>(n) * p.prev_stride], 0, V - 1);
  const float u_raw = p.u_draft[o];
  const int per_w = (n_seg + NW - 1) / NW;
  const int w0 = wave * per_w;
  const int n_w = max(0, min(per_w, n_seg - w0));
  const int L = (n_w + 63) >> 6;  // wavefront-uniform, <= J
  float2 r[J];
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < L) r[j] = rec[w0 + min(j * 64 + lane, n_w - 1)];
  HRow<WT, NT> hrow;
  if (p.hstate != nullptr)
    hrow.hold_state(p.hstate + o * p.rank, p.rank);
  else
    hrow.hold(static_cast<const WT*>(p.W1), prev, p.rank);
  // the RNN head's next state in this finish (workgroup-uniform): its z
  // (rank <= DSPARK_MAX_RANK <= NT values), loaded with the records
  const bool fuse = SEG == kSegSmall && p.A != nullptr && p.k + 1 < p.gamma;
  static_assert(DSPARK_MAX_RANK <= NT || SEG != kSegSmall, "one state value per thread");
  const float zj = (fuse && tid < p.rank) ? p.hstate[(o + 1) * p.rank + tid] : 0.0f;
  const float c = temp_scale(T);  // the same for the whole workgroup
  const bool greedy = c == 0.0f;
  // records past the wavefront's range: no mass, never the maximum
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < L) {
      const bool in = j * 64 + lane < n_w;
      r[j].x = in ? r[j].x : -INFINITY;
      r[j].y = in ? r[j].y : (greedy ? __int_as_float(kIntMax) : 0.0f);
    }
  }
  if (greedy) {
    // the records carry their lowest argmax in the second word
    float m = -INFINITY;
    int im = kIntMax;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < L) amax_merge(m, im, r[j].x, __float_as_int(r[j].y));
    wave_amax(m, im);
    if (lane == 0) {
      sm.wm[wave] = m;
      sm.wi[wave] = im;
    }
    __syncthreads();
    // wavefront 0 (with the fused state, every wavefront) combines the pairs
    if (wave == 0 || fuse) {
      m = lane < NW ? sm.wm[lane] : -INFINITY;
      im = lane < NW ? sm.wi[lane] : kIntMax;
      wave_amax(m, im);
      if (wave == 0 && lane == 0) {
        p.y[o] = clampi(im, 0, V - 1);
        p.q_tok[o] = 1.0f;
        p.q_stats[2 * o] = m;
        p.q_stats[2 * o + 1] = 1.0f;
      }
      if (fuse) fused_state_store(p, zj, im, o);
    }
    return;
  }
  // sampled: the wavefront's maximum and its mass sum relative to it
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < L) m = fmaxf(m, r[j].x);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j < L) s += r[j].y * exp2_rel(r[j].x, m, c);
  s = wave_sum(s);
  hrow.commit(p.rank, sm.hs);
  if (lane == 0) {
    sm.wm[wave] = m;
    sm.ws[wave] = s;
  }
  __syncthreads();
  // every wavefront, lane w holding wavefront w's pair: M, the masses in
  // units of 2^((. - M) c), their inclusive prefix and Z; the wavefront
  // whose interval holds theta = u Z, else the last one with mass (the
  // fallback that takes the last positive entry)
  const float mw = lane < NW ? sm.wm[lane] : -INFINITY;
  const float sw = lane < NW ? sm.ws[lane] : 0.0f;
  float M = mw;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  const float S = sw * exp2_rel(mw, M, c);
  const float incl = wave_incl_scan(S);
  const float iup = __shfl_up(incl, 1);
  const float excl = (lane == 0) ? 0.0f : iup;  // [excl, incl) of consecutive lanes meet exactly
  const float Z = readlane_f(incl, 63);
  const float theta = clamp_uniform(u_raw) * Z;
  const unsigned long long whit = __ballot(S > 0.0f && incl > theta);
  const unsigned long long wpos = __ballot(S > 0.0f);
  bool fb = whit == 0;
  const int wfin = whit ? (__ffsll(static_cast<long long>(whit)) - 1)
                        : (wpos ? 63 - __clzll(static_cast<long long>(wpos)) : 0);
  if (wave == wfin) draft_finish_waves_pick<WT, NT, J, SEG>(p, sm, r, n, o, w0, L, M, Z, c, theta,
                                                             readlane_f(excl, wfin), fb);
  if (fuse) {
    __syncthreads();  // the chosen wavefront's token
    fused_state_store(p, zj, sm.ynext, o);
  }
  if constexpr (SEG == kSegWide) {
    __syncthreads();
    draft_finish_rescan64<WT, NT>(p, sm, n, o, M, Z, c);
  }
}

}  // namespace dspark
