// Single-GEMM kernels, weight loads with cache policy "sc1".
#include "gemm_instances.h"

namespace sg {
GemmKernel gemm_kernel_sc1(int path, int a, int b) { return gemm_kernel_for<(kAuxNt | kAuxSc1)>(path, a, b); }
}  // namespace sg
