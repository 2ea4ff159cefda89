// Single-GEMM kernels, weight loads with cache policy "cached".
#include "gemm_instances.h"

namespace sg {
GemmKernel gemm_kernel_cached(int path, int a, int b) { return gemm_kernel_for<0>(path, a, b); }
}  // namespace sg
