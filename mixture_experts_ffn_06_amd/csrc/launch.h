// Host-side, one-time launch set-up shared by the kernel launchers.
//
// Each launcher keeps its set-up in a function-local static initialised by
// these helpers: C++ runs such an initialiser exactly once even when several
// host threads make their first call together, so the library stays safe to
// call from several threads (a plan is immutable; each call brings its own
// workspace).  A failed set-up is kept and returned on every later call.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

struct KernelSetup {
  hipError_t err;
  int blocks_per_cu;   // resident blocks of the kernel per CU at that LDS size
};

// Allow lds_bytes of dynamic LDS for kern and find how many blocks of
// `threads` fit one CU.
inline KernelSetup kernel_setup(const void *kern, int threads, int lds_bytes) {
  KernelSetup r{hipSuccess, 0};
  r.err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (r.err != hipSuccess) return r;
  r.err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&r.blocks_per_cu, kern, threads, lds_bytes);
  if (r.err == hipSuccess && r.blocks_per_cu < 1) r.err = hipErrorInvalidConfiguration;
  return r;
}

// Only the dynamic-LDS allowance (kernels launched as single blocks).
inline hipError_t lds_setup(const void *kern, int lds_bytes) {
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
}

// Compute units of the current device at the first call (every device the
// process uses is taken to be alike; 256 if the query fails).
inline int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

}  // namespace moe
