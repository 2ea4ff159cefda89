// Single-GEMM kernels, weight loads with cache policy "nt".
#include "gemm_instances.h"

namespace sg {
GemmKernel gemm_kernel_nt(int path, int a, int b) { return gemm_kernel_for<kAuxNt>(path, a, b); }
}  // namespace sg
