// Whole decoder layer in one persistent launch: launch and instantiations
// (the kernel is in decoder_body.h).  MFMA stages for MT = 1..4 m-tiles with
// one or two n-tiles (two only up to two m-tiles, as the chain), dot2 stages
// for M = 1 and 2 with G = 2 or 4 weight rows per wave.
#include <hip/hip_runtime.h>

#include "decoder_body.h"

namespace sg {

static ChainKernel decoder_kernel(int path, int a, int b) {
  if (path == 0) {
    switch (a * 8 + b) {
      case 1 * 8 + 2: return k_decoder<0, 1, 2>;
      case 1 * 8 + 4: return k_decoder<0, 1, 4>;
      case 2 * 8 + 2: return k_decoder<0, 2, 2>;
      case 2 * 8 + 4: return k_decoder<0, 2, 4>;
      default: return nullptr;
    }
  }
  switch (a * 4 + b) {
    case 1 * 4 + 1: return k_decoder<1, 1, 1>;
    case 1 * 4 + 2: return k_decoder<1, 1, 2>;
    case 2 * 4 + 1: return k_decoder<1, 2, 1>;
    case 2 * 4 + 2: return k_decoder<1, 2, 2>;
    case 3 * 4 + 1: return k_decoder<1, 3, 1>;
    case 4 * 4 + 1: return k_decoder<1, 4, 1>;
    default: return nullptr;
  }
}

bool decoder_variant_exists(int path, int a, int b) { return decoder_kernel(path, a, b) != nullptr; }

hipError_t launch_decoder(const ChainArgs& a, int grid, int block, int lds, hipStream_t stream) {
  ChainKernel k = decoder_kernel(a.path, a.mt, a.nt_q);
  if (!k) return hipErrorInvalidValue;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(block), lds, stream, a);
  return hipGetLastError();
}

}  // namespace sg
