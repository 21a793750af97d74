// Causal prefix-closed global top-K verify scheduler ("DSpark" explainer
// sections 4, 5, 8-10 and 13), and the static confidence cutoff (Strata
// plan "Approach" step 5; llama.cpp PR #25173 "Confidence Evaluation",
// conf_min), which replaces the top-K selection by a per-request rule: the
// leading positions whose own clamped confidence is at least conf_min.
//
// One workgroup of 1024 threads.  Thread t owns requests t, t + 1024, ...;
// their survival values a[r, k] (fp32 running product of the clamped c) live
// in registers as 64-bit keys (~bits(a) << 32 | k << 24 | r), whose ascending
// order is (a descending, k ascending, r ascending).  The Kc-th smallest key is
// found by an 8-pass radix select (8-bit digits, LDS histograms); a candidate
// is selected iff its key is <= that threshold, which gives exactly Kc
// selections.  The last four passes (the (k, r) tie-break) are skipped when
// the survival bits alone leave a bucket whose members are all selected.
// Then l[r], an exclusive scan of l[r] + 1 for the row offsets, and the
// flattened rows.  Nothing here reads the drafted tokens except the
// copy into row_tok.

#include "dspark_device.h"
#include "launchers.h"

namespace dspark {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSlots = DSPARK_SCHED_KEYS_PER_THREAD;

__device__ __forceinline__ int wave_excl_scan_int(int v, int* total) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(x, d);
    if (lane >= d) x += o;
  }
  *total = __shfl(x, 63);
  return x - v;
}

// exclusive scan over the 1024 threads; returns excl, *total = block sum
__device__ __forceinline__ int block1024_excl_scan_int(int v, int* lds16, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int wt;
  const int ex = wave_excl_scan_int(v, &wt);
  if (lane == 0) lds16[wave] = wt;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int x = lds16[w];
    if (w < wave) off += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + ex;
}

template <bool CUTOFF>
__global__ void __launch_bounds__(kSchedThreads) schedule_kernel(dspark_schedule_args a, float conf_min) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_rem;
  __shared__ int s_all;
  __shared__ int s_i16[16];
  __shared__ float s_f16[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.R, gamma = a.gamma;
  const int JR = (R + kSchedThreads - 1) / kSchedThreads;
  const int used = JR * gamma;

  unsigned long long key[kSlots];
  bool valid[kSlots];
  bool keep[kSlots];  // static cutoff: position still inside the request's leading run
  // the confidences and drafted tokens of this thread's slots are loaded up
  // front, in one batch
  float cv[kSlots];
  int yv[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int j = s / gamma, k = s - j * gamma;
    const int r = j * kSchedThreads + tid;
    valid[s] = (s < used) && (r < R);
    const int64_t o = valid[s] ? static_cast<int64_t>(r) * gamma + k : 0;
    cv[s] = valid[s] ? a.c[o] : 0.0f;
    yv[s] = valid[s] ? a.y[o] : 0;
  }
  float run = 1.0f;
  bool alive = true;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int j = s / gamma, k = s - j * gamma;
    const int r = j * kSchedThreads + tid;
    key[s] = ~0ull;
    keep[s] = false;
    if (valid[s]) {
      const int64_t o = static_cast<int64_t>(r) * gamma + k;
      float ck = fminf(fmaxf(cv[s], 0.0f), 1.0f);  // NaN -> 0
      run = (k == 0) ? ck : run * ck;
      alive = ((k == 0) || alive) && (ck >= conf_min);
      keep[s] = alive;
      const float av = (run == 0.0f) ? 0.0f : run;  // no -0
      a.a[o] = av;
      const unsigned int bits = __float_as_uint(av);
      key[s] = (static_cast<unsigned long long>(~bits) << 32) | (static_cast<unsigned long long>(k) << 24) |
               static_cast<unsigned long long>(r);
    }
  }

  const int64_t n = static_cast<int64_t>(R) * gamma;
  const int64_t Kc = a.K < 0 ? 0 : (a.K > n ? n : a.K);
  unsigned long long thr = 0;
  bool none = (Kc == 0), all = (Kc == n);
  if (!CUTOFF && !none && !all) {
    unsigned long long prefix = 0;
    int rem = static_cast<int>(Kc);
    int pass = 0;
    for (; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        if (valid[s] && (pass == 0 || (key[s] >> (shift + 8)) == (prefix >> (shift + 8))))
          atomicAdd(&hist[(key[s] >> shift) & 255ull], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        int tot;
        const int ex = wave_excl_scan_int(h0 + h1 + h2 + h3, &tot);
        if (ex < rem && rem <= ex + h0 + h1 + h2 + h3) {
          const int hs[4] = {h0, h1, h2, h3};
          int cb = ex;
          for (int q = 0; q < 4; ++q) {
            if (rem <= cb + hs[q]) {
              s_prefix = prefix | (static_cast<unsigned long long>(4 * lane + q) << shift);
              s_rem = rem - cb;
              s_all = (rem - cb == hs[q]) ? 1 : 0;
              break;
            }
            cb += hs[q];
          }
        }
      }
      __syncthreads();
      prefix = s_prefix;
      rem = s_rem;
      // once the survival bits are fixed (the upper 32), a threshold bucket
      // whose every member is selected needs no tie-break by (k, r): all
      // keys up to the bucket's largest are taken (uniform: read from LDS)
      if (pass == 3 && s_all) break;
    }
    thr = (pass < 8) ? (prefix | 0xFFFFFFFFull) : prefix;
  }

  // l[r] and this thread's contribution to the expected token count
  int lj[kSlots];  // l per owned request (indexed by j), kept in the first JR slots
  float esum = 0.0f;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) lj[s] = 0;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    if (valid[s]) {
      const bool sel = CUTOFF ? keep[s] : (all || (!none && key[s] <= thr));
      if (sel) {
        const int j = s / gamma;
#pragma unroll
        for (int q = 0; q < kSlots; ++q)
          if (q == j) lj[q] += 1;
        esum += __uint_as_float(~static_cast<unsigned int>(key[s] >> 32));
      }
    }
  }

  // row offsets: exclusive scan of l[r] + 1 in request order (round j covers
  // requests j*1024 .. j*1024+1023)
  int carry = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (j < JR) {
      const int r = j * kSchedThreads + tid;
      const int cnt = (r < R) ? lj[j] + 1 : 0;
      const int anc = (r < R) ? a.anchor[r] : 0;  // in flight during the scan
      int tot;
      const int ex = block1024_excl_scan_int(cnt, s_i16, &tot);
      if (r < R) {
        const int off = carry + ex;
        a.l[r] = lj[j];
        a.row_offsets[r] = off;
        // row pos of request r: the anchor for pos 0, else y[r, pos - 1]
        // (slot j * gamma + pos - 1 of this thread)
#pragma unroll
        for (int q = 0; q <= kSlots; ++q) {
          if (q <= lj[j]) {
            int tok = anc;
#pragma unroll
            for (int s = 0; s < kSlots; ++s) tok = (q >= 1 && s == j * gamma + q - 1) ? yv[s] : tok;
            a.row_req[off + q] = r;
            a.row_pos[off + q] = q;
            a.row_tok[off + q] = tok;
          }
        }
      }
      carry += tot;
    }
  }
  if (tid == 0) a.row_offsets[R] = carry;

  if (a.expected_tokens != nullptr) {
    esum = wave_sum(esum);
    if (lane == 0) s_f16[wave] = esum;
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f;
      for (int w = 0; w < 16; ++w) t += s_f16[w];
      a.expected_tokens[0] = static_cast<float>(R) + t;
    }
  }
}

}  // namespace

hipError_t launch_schedule(const dspark_schedule_args& a, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  hipLaunchKernelGGL(schedule_kernel<false>, dim3(1), dim3(kSchedThreads), 0, s, a, 0.0f);
  return hipGetLastError();
}

hipError_t launch_schedule_cutoff(const dspark_schedule_args& a, float conf_min, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  hipLaunchKernelGGL(schedule_kernel<true>, dim3(1), dim3(kSchedThreads), 0, s, a, conf_min);
  return hipGetLastError();
}

}  // namespace dspark
