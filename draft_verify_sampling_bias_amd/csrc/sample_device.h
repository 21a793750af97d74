// Inverse-CDF location over per-segment partial sums, shared by the finish
// kernels (256 threads per workgroup, one request per workgroup).
//
// An inverse-CDF draw walks the vocabulary in index order and returns the
// first entry whose inclusive cumulative mass exceeds u * Z.  The vocabulary
// is covered by segments whose masses were reduced by an earlier kernel, so
// the walk is done in levels: block-wide prefixes over segment masses pick
// the segment, and only that segment's 16 or 32 entries are recomputed
// and scanned (a target row, which is an input, is rescanned in chunks of
// 4096 entries instead).  Intervals of
// consecutive threads meet exactly (block256_scan), so exactly one thread owns
// any threshold; where rounding between levels leaves the threshold past the
// last entry of a chosen range, the last positive-mass entry of that range is
// returned (zero-mass entries are never returned).
#pragma once

#include "dspark_device.h"
#include "plan.h"

namespace dspark {

struct LocScratch {
  float scan[4];
  float fred[4];
  int ired[4];
  int sel;
  float P;
};

struct Located {
  int index;       // selected segment (-1 if no mass at all)
  float P;         // cumulative mass before it
  float Z;         // total mass
  bool fallback;   // threshold fell past the end: take the last positive entry
};

__device__ __forceinline__ float clamp_uniform(float u) {
  // [0, 1); NaN -> 0
  return fminf(fmaxf(u, 0.0f), 0x1.fffffep-1f);
}

// Block-wide location over `n` segments with masses mass(t) >= 0 at threshold
// u * Z.  Each thread sums a contiguous run of segments.
template <class Mass>
__device__ Located locate_segments(int n, Mass mass, float u, LocScratch* sh) {
  const int tid = threadIdx.x;
  const int seg = (n + 255) / 256;
  const int t0 = min(tid * seg, n), t1 = min(t0 + seg, n);
  float ts = 0.0f;
  int lastpos = -1;
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {
    const float x = mass(t);
    ts += x;
    if (x > 0.0f) lastpos = t;
  }
  float excl, Z;
  const float incl = block256_scan(ts, sh->scan, &excl, &Z);
  const float theta = u * Z;
  const int first = block256_min_int((incl > theta) ? tid : 256, sh->ired);
  const int glast = block256_max_int(lastpos, sh->ired);
  if (tid == first) {
    float run = excl;
    int found = -1;
    float P = excl, Plast = excl;
    int seglast = -1;
    for (int t = t0; t < t1; ++t) {
      const float x = mass(t);
      const float nx = run + x;
      if (x > 0.0f) {
        seglast = t;
        Plast = run;
        if (nx > theta) {
          found = t;
          P = run;
          break;
        }
      }
      run = nx;
    }
    sh->sel = (found >= 0) ? found : -(seglast + 2);  // encode "segment fallback"
    sh->P = (found >= 0) ? P : Plast;
  }
  __syncthreads();
  Located L;
  L.Z = Z;
  L.fallback = false;
  if (first < 256) {
    const int s = sh->sel;
    if (s >= 0) {
      L.index = s;
      L.P = sh->P;
    } else {
      L.index = -(s + 2);
      L.P = sh->P;
      L.fallback = true;
    }
  } else {
    L.index = glast;
    L.P = 0.0f;
    L.fallback = true;
  }
  __syncthreads();
  return L;
}

// Two-level location over n segment masses mass(t) >= 0: thread i sums the
// contiguous block i of a balanced 256-way partition, a block-wide scan
// picks the block whose interval holds u * Z, and wavefront 0 scans that
// block's masses 64 at a time to pick the segment.  Returns the segment and
// the threshold left inside it (same units as the masses), or fallback =
// true (threshold INFINITY: take the segment's last positive entry) when
// rounding between the levels leaves the threshold past the block's last
// positive segment, or when no block's interval holds it.  seg = -1 when
// every mass is zero.  All threads get the result.
struct Located2 {
  int seg;
  float rem;
  float Z;
  bool fallback;
};

constexpr int kLocMaxWaves = 16;  // workgroups of up to 1024 threads
struct Loc2Scratch {
  float wsum[kLocMaxWaves];   // per-wavefront totals of the block scan
  float fred[kLocMaxWaves];   // per-wavefront maxima (finish kernels)
  int ired[kLocMaxWaves];
  int cand[kLocMaxWaves];     // per-wavefront first thread whose interval holds u Z
  float cexcl[kLocMaxWaves];  // and its exclusive prefix
  int glast[kLocMaxWaves];    // per-wavefront last segment with positive mass
  int sel;
  float rem;
  int fb;
};

// First segment of thread block i of the NT-way partition.
template <int NT = 256>
__device__ __forceinline__ int block_begin(int i, int n) { return range_start(i, n, NT); }

// Second half of the location: ts is this thread's block sum (already in
// the units of mass()), lastpos its last segment with positive mass (or -1).
// Three workgroup barriers; every scratch slot is written once per call, so
// no barrier is needed to protect reuse (callers must not call it twice
// with the same scratch without a barrier in between).
template <int NT = 256, class Mass>
__device__ Located2 locate_from_block_sums(int n, float ts, int lastpos, Mass mass, float u, Loc2Scratch* sh) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // block-wide scan: thread intervals [excl, incl) of consecutive threads
  // meet exactly (incl of one thread is excl of the next, bit for bit: every
  // wavefront offset is the same left-to-right sum of the totals before it)
  const float v = wave_incl_scan(ts);
  if (lane == 63) sh->wsum[wave] = v;
  __syncthreads();
  float off = 0.0f, Z = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float x = sh->wsum[w];
    off = (w < wave) ? Z + x : off;
    Z += x;
  }
  const float incl = off + v;
  const float up = __shfl_up(incl, 1);
  const float excl = (lane == 0) ? off : up;
  const float theta = u * Z;
  // the first thread whose interval holds theta, with its exclusive prefix,
  // and the last positive segment, in one barrier round
  const unsigned long long hit = __ballot(incl > theta);
  const int fl = hit ? (__ffsll(static_cast<long long>(hit)) - 1) : 0;
  const float fex = __shfl(excl, fl);
  const int wl = wave_max_int(lastpos);
  if (lane == 0) {
    sh->cand[wave] = hit ? (wave * 64 + fl) : NT;
    sh->cexcl[wave] = fex;
    sh->glast[wave] = wl;
  }
  __syncthreads();
  int first = NT;
  float P = 0.0f;
  int glast = -1;
#pragma unroll
  for (int w = NW - 1; w >= 0; --w) {
    const bool has = sh->cand[w] < NT;
    first = has ? sh->cand[w] : first;
    P = has ? sh->cexcl[w] : P;
    glast = max(glast, sh->glast[w]);
  }
  int s0, s1;
  float th;
  bool fb;
  if (first < NT) {
    s0 = block_begin<NT>(first, n);
    s1 = block_begin<NT>(first + 1, n);
    th = theta - P;
    fb = false;
  } else {
    s0 = max(glast, 0);
    s1 = glast + 1;
    th = INFINITY;
    fb = true;
  }
  if (tid < 64) {
    int sel = -1, lpos = -1;
    float selP = 0.0f, lastP = 0.0f, base = 0.0f;
    for (int c0 = s0; c0 < s1; c0 += 64) {
      const int sidx = c0 + lane;
      const float x = (sidx < s1) ? mass(sidx) : 0.0f;
      const float cum = wave_incl_scan(x);
      const float cup = __shfl_up(cum, 1);
      const float ex = (lane == 0) ? 0.0f : cup;
      const unsigned long long h2 = __ballot(x > 0.0f && base + cum > th);
      const unsigned long long pos = __ballot(x > 0.0f);
      if (pos) {
        const int lp = 63 - __clzll(static_cast<long long>(pos));
        lpos = c0 + lp;
        lastP = base + __shfl(ex, lp);
      }
      if (h2) {
        const int f2 = __ffsll(static_cast<long long>(h2)) - 1;
        sel = c0 + f2;
        selP = base + __shfl(ex, f2);
        break;
      }
      base += __shfl(cum, 63);
    }
    bool f = fb;
    if (sel < 0) {
      sel = lpos;
      selP = lastP;
      f = true;
    }
    if (lane == 0) {
      sh->sel = sel;
      sh->rem = f ? INFINITY : th - selP;
      sh->fb = f ? 1 : 0;
    }
  }
  __syncthreads();
  Located2 out;
  out.seg = sh->sel;
  out.rem = sh->rem;
  out.fallback = sh->fb != 0;
  out.Z = Z;
  return out;
}

template <int NT = 256, class Mass>
__device__ Located2 locate_blocked(int n, Mass mass, float u, Loc2Scratch* sh) {
  const int tid = threadIdx.x;
  const int t0 = block_begin<NT>(tid, n), t1 = block_begin<NT>(tid + 1, n);
  float ts = 0.0f;
  int lastpos = -1;
#pragma unroll 8
  for (int t = t0; t < t1; ++t) {
    const float x = mass(t);
    ts += x;
    lastpos = (x > 0.0f) ? t : lastpos;
  }
  return locate_from_block_sums<NT>(n, ts, lastpos, mass, u, sh);
}

// Wave 0: first of n <= 64 weights whose inclusive prefix exceeds theta,
// else the last positive one, else -1.
__device__ __forceinline__ int pick64_reg(float x, float theta) {
  const float cum = wave_incl_scan(x);
  const unsigned long long hit = __ballot(x > 0.0f && cum > theta);
  if (hit) return __ffsll(static_cast<long long>(hit)) - 1;
  const unsigned long long pos = __ballot(x > 0.0f);
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : -1;
}
__device__ __forceinline__ int pick64(const float* e, int n, float theta) {
  const int lane = threadIdx.x & 63;
  return pick64_reg((lane < n) ? e[lane] : 0.0f, theta);
}

// The draw inside the chosen segment from the rows' logits as a rescan
// recomputes them (lane i: row i of n <= 64, -inf where masked), by a whole
// wavefront.  Those logits can differ from the ones the segment records were
// built from by rounding (fp32 weights summed in another order than the
// fused kernel's), and a large scale c (a tiny temperature) turns such a
// difference into 2^(+-huge) when it is measured against the record's
// maximum.  The weights are therefore taken relative to the rescan's own
// maximum, where the top row weighs exactly 1, and the draw uses the rescan's
// own total with the fraction frac of the segment's mass that the search over
// the records left over.  With logits identical to the records' the draw is
// the one against the records.  Returns the row (-1: no positive weight) and
// its probability within the segment.
struct SegPick {
  int pos;
  float qin;
};
__device__ __forceinline__ SegPick seg_pick_own_max(float sv, int n, float c, float frac) {
  const int lane = threadIdx.x & 63;
  if (lane >= n) sv = -INFINITY;
  // maximum over the lanes that hold rows (lanes past n keep -inf and
  // weight 0 whatever they see)
  float mr = sv;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1)
    if (d < n) mr = fmaxf(mr, __shfl_xor(mr, d));
  const float e = (sv == -INFINITY) ? 0.0f : exp2_rel(sv, mr, c);
  // the inclusive scan gives the total at lane 63, then the pick as in pick64
  const float cum = wave_incl_scan(e);
  const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 63));
  const unsigned long long hit = __ballot(e > 0.0f && cum > frac * tot);
  const unsigned long long any = __ballot(e > 0.0f);
  const int pos = hit ? (__ffsll(static_cast<long long>(hit)) - 1)
                      : (any ? 63 - __clzll(static_cast<long long>(any)) : -1);
  const float ey = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), pos < 0 ? 0 : pos));
  return SegPick{pos, (pos >= 0 && tot > 0.0f) ? ey / tot : 0.0f};
}

// Eight consecutive weights of a row, loaded raw, and their product with h
// (fp32 accumulate, fixed order).
struct Raw8 {
  u32x4_t a, b;  // bf16: 8 weights in a; fp32: 4 + 4
};
__device__ __forceinline__ Raw8 load8(const uint16_t* row, int k) {
  return Raw8{*reinterpret_cast<const u32x4_t*>(row + k), u32x4_t{0u, 0u, 0u, 0u}};
}
__device__ __forceinline__ Raw8 load8(const float* row, int k) {
  return Raw8{*reinterpret_cast<const u32x4_t*>(row + k), *reinterpret_cast<const u32x4_t*>(row + k + 4)};
}
__device__ __forceinline__ float dot8(const Raw8& r, const uint16_t*, const float* h, int k) {
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(__uint_as_float(r.a[q] << 16), h[k + 2 * q], acc);
    acc = fmaf(__uint_as_float(r.a[q] & 0xffff0000u), h[k + 2 * q + 1], acc);
  }
  return acc;
}
__device__ __forceinline__ float dot8(const Raw8& r, const float*, const float* h, int k) {
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(r.a[q]), h[k + q], acc);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(r.b[q]), h[k + 4 + q], acc);
  return acc;
}

// Markov bias W2[v, :] . h for one vocabulary row per group of 2^lpr_log2
// consecutive lanes (row index = threadIdx.x >> lpr_log2, lpr_log2 >= 2).
// Every lane of the group returns the same value.  A lane's weight loads are
// all issued before any is used (at most DSPARK_MAX_RANK / 32 of them).
// MIN_LG: a lower bound of lpr_log2 known at compile time (bounds the
// number of weight chunks a lane can hold, and so its registers).
template <typename WT, int MIN_LG = 2>
__device__ __forceinline__ float row_bias(const WT* W2, const float* hs, int rank, int v, int V, int lpr_log2) {
  constexpr int kMaxChunks = DSPARK_MAX_RANK / (8 << MIN_LG);
  const int lpr = 1 << lpr_log2;
  const int part = threadIdx.x & (lpr - 1);
  const WT* row = W2 + static_cast<int64_t>(min(v, V - 1)) * rank;
  // chunk it exists for some lane of the group iff it * lpr * 8 < rank
  // (wavefront-uniform: a scalar branch)
  Raw8 r[kMaxChunks];
#pragma unroll
  for (int it = 0; it < kMaxChunks; ++it) {
    const int k = (part + it * lpr) * 8;
    if (it * lpr * 8 < rank) r[it] = load8(row, min(k, rank - 8));
  }
  float acc = 0.0f;
#pragma unroll
  for (int it = 0; it < kMaxChunks; ++it) {
    const int k = (part + it * lpr) * 8;
    if (it * lpr * 8 < rank && k < rank) acc += dot8(r[it], row, hs, k);
  }
  for (int d = 1; d < lpr; d <<= 1) acc += __shfl_xor(acc, d);
  return (v < V) ? acc : 0.0f;
}

template <typename WT>
__device__ __forceinline__ float weight_at(const WT* w, int64_t i);
template <>
__device__ __forceinline__ float weight_at<uint16_t>(const uint16_t* w, int64_t i) {
  return bf16_to_f32(w[i]);
}
template <>
__device__ __forceinline__ float weight_at<float>(const float* w, int64_t i) {
  return w[i];
}

// h = W1[prev, :] as fp32 into LDS (no barrier).
template <typename WT>
__device__ __forceinline__ void load_h(const WT* W1, int prev, int rank, float* hs) {
  for (int k = threadIdx.x; k < rank; k += 256) hs[k] = weight_at<WT>(W1, static_cast<int64_t>(prev) * rank + k);
}

struct ChunkScratch {
  LocScratch loc;
  float scan[4];
  int ired[4];
};

// Inverse-CDF draw with uniform u from p ~ exp((t - M)/T) over one target row,
// using the row's per-chunk records (max, argmax, sum of exp2((t - max) c)).
// Returns the token (all threads), or -1 if the row has no mass.
__device__ __forceinline__ int chunk_draw(const float* vrec, int n_chunks, const float* __restrict__ trow, int V,
                                          float M, float c, float u, ChunkScratch* sh) {
  auto mass = [&](int ch) { return vrec[ch * kChunkFloats + 2] * exp2_hw((vrec[ch * kChunkFloats] - M) * c); };
  const Located L = locate_segments(n_chunks, mass, u, &sh->loc);
  if (L.index < 0) return -1;
  const int ch = L.index;
  const float mc = vrec[ch * kChunkFloats];
  const float scale = exp2_hw((mc - M) * c);
  const float th = L.fallback ? INFINITY : (u * L.Z - L.P) / scale;
  const int tid = threadIdx.x;
  const int v0 = ch * kChunk + tid * 16;
  float e[16];
  float ts = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int v = v0 + j;
    e[j] = (v < V) ? exp2_hw((trow[v] - mc) * c) : 0.0f;
    ts += e[j];
  }
  float excl, tot;
  const float incl = block256_scan(ts, sh->scan, &excl, &tot);
  int cand = kIntMax, lastpos = -1;
  if (incl > th) {
    float run = excl;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float nx = run + e[j];
      if (cand == kIntMax && e[j] > 0.0f && nx > th) cand = v0 + j;
      run = nx;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (e[j] > 0.0f) lastpos = v0 + j;
  // the first thread whose interval reaches th owns the answer
  const int first = block256_min_int(cand, sh->ired);
  if (first != kIntMax) return first;
  return block256_max_int(lastpos, sh->ired);
}

}  // namespace dspark
