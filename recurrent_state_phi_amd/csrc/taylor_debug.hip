// Test hook: fill the LDS of every CU with a given 32-bit pattern, so that a
// kernel launched next on the same stream starts from LDS holding that pattern
// (the hardware leaves LDS as the previous workgroup left it).  A kernel that
// reads LDS before writing it then computes with the pattern (for example NaN),
// and its results no longer match the oracle.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "taylor_launch.h"

namespace taylor {
namespace debug {

// Nearly all of a CU's 160 KB, so that one such workgroup fills a CU's LDS and
// no other workgroup of this kernel shares the CU while it runs.
constexpr int kFillWords = (160 * 1024 - 1024) / 4;

__global__ __launch_bounds__(1024) void fill_lds_kernel(uint32_t pattern) {
  __shared__ uint32_t lds[kFillWords];
  // LDS stores the compiler must keep (nothing reads them in this kernel)
  volatile __attribute__((address_space(3))) uint32_t* p = (__attribute__((address_space(3))) uint32_t*)lds;
  for (int i = threadIdx.x; i < kFillWords; i += 1024) p[i] = pattern;
  __syncthreads();
}

}  // namespace debug

hipError_t launch_fill_lds(uint32_t pattern, hipStream_t stream) {
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return e;
  // two rounds of one workgroup per CU, so that every CU gets at least one
  hipLaunchKernelGGL(debug::fill_lds_kernel, dim3(2 * cus), dim3(1024), 0, stream, pattern);
  return hipGetLastError();
}

}  // namespace taylor
