// Host-side facts about the current HIP device, queried once per device.
#pragma once

#include <hip/hip_runtime.h>

namespace dspark {

// Compute units of the current device (persistent-grid and workgroup-size
// choices), cached per device; 256 if the query fails.
inline int current_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

}  // namespace dspark
