// Persistent layer chain: launch and the MFMA-stage instantiations (the
// kernel itself is in chain_body.h).
#include <hip/hip_runtime.h>

#include "chain_body.h"

namespace sg {

static ChainKernel chain_kernel(int path, int a, int b) {
  if (path == 0) return chain_kernel_dot2(a, b);
  if (path == 3) return chain_kernel_kc(a, b);
  switch (a * 4 + b) {
    case 1 * 4 + 1: return k_chain<1, 1, 1>;
    case 1 * 4 + 2: return k_chain<1, 1, 2>;
    case 2 * 4 + 1: return k_chain<1, 2, 1>;
    case 2 * 4 + 2: return k_chain<1, 2, 2>;
    case 3 * 4 + 1: return k_chain<1, 3, 1>;
    case 4 * 4 + 1: return k_chain<1, 4, 1>;
    default: return nullptr;
  }
}

bool chain_variant_exists(int path, int a, int b) {
  // MFMA: MT >= 3 with two n-tiles in the unpaired stages does not fit the
  // register file next to the paired gate_up stage (it spills), so it is not
  // offered.
  if (path == 1 && a >= 3 && b == 2) return false;
  return chain_kernel(path, a, b) != nullptr;
}

hipError_t launch_chain(const ChainArgs& a, int grid, int block, int lds, hipStream_t stream) {
  ChainKernel k = chain_kernel(a.path, a.mt, a.nt_q);
  if (!k) return hipErrorInvalidValue;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(block), lds, stream, a);
  return hipGetLastError();
}

}  // namespace sg
