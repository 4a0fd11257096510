// occupancy.hpp -- host-side occupancy caps for the streaming launches.
//
// A launch of 256-thread blocks (one wave per SIMD each) can be held to at
// most `bpc` resident blocks per compute unit by giving every block an equal
// share of the unit's LDS as dynamic shared memory, which the kernels do not
// use.  On this HBM some streaming kernels run faster with fewer waves in
// flight than their registers allow; the caps in use are measured per kernel.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>

namespace oba {

// Dynamic LDS bytes per block for a cap of bpc blocks per CU (0: no cap).  A
// 4 KB margin leaves room for each kernel's static LDS, so bpc blocks fit
// and bpc + 1 do not.
inline size_t occupancy_lds(int bpc) {
  if (bpc <= 0) return 0;
  constexpr int kDevs = 64;
  static std::atomic<int> per_cu_cache[kDevs];  // LDS bytes per CU, 0 = not yet read
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  int per_cu = per_cu_cache[dev].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        per_cu <= 0)
      return 0;
    per_cu_cache[dev].store(per_cu, std::memory_order_relaxed);
  }
  const size_t share = (size_t)(per_cu / bpc) / 512 * 512;
  return share > 4096 ? share - 4096 : 0;
}

// Shares above 64 KB must be allowed per kernel.
inline void allow_lds(const void* kernel, size_t lds) {
  if (lds > 65536)
    (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace oba
