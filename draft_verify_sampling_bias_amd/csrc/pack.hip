// W2 rearranged into the fragment-packed layout of the 16-row fused bias
// kernel (include/dspark.h, dspark_pack_w2): one thread per 16-byte slot,
// coalesced writes.  A one-time step at model load.

#include "dspark_device.h"
#include "launchers.h"
#include "plan.h"

namespace dspark {
namespace {

__global__ void __launch_bounds__(256) pack_w2_kernel(const uint16_t* __restrict__ W2, uint16_t* __restrict__ out,
                                                      int V, int rank, int ks_count, int64_t n_slots) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_slots) return;
  const int L = static_cast<int>(t & 63);
  const int64_t sk = t >> 6;  // s * KS + ks
  const int ks = static_cast<int>(sk % ks_count);
  const int64_t s = sk / ks_count;
  const int64_t v = 16 * s + (L & 15);
  const int k = 32 * ks + 8 * (L >> 4);
  u32x4_t val{0u, 0u, 0u, 0u};
  if (v < V && k < rank) val = *reinterpret_cast<const u32x4_t*>(W2 + v * rank + k);
  *reinterpret_cast<u32x4_t*>(out + t * 8) = val;
}

}  // namespace

hipError_t launch_pack_w2(const dspark_pack_w2_args& a, hipStream_t s) {
  const int ks_count = seg16_ksteps(a.rank);
  const int64_t n_slots = static_cast<int64_t>((a.V + 15) / 16) * ks_count * 64;
  const int64_t blocks = (n_slots + 255) / 256;
  hipLaunchKernelGGL(pack_w2_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(a.W2), static_cast<uint16_t*>(a.W2_packed), a.V, a.rank,
                     ks_count, n_slots);
  return hipGetLastError();
}

}  // namespace dspark
