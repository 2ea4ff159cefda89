// Launch of the single-GEMM kernels (one launch per sgemm_run), the
// workspace fill kernel and the XCD topology probe.
#include <hip/hip_runtime.h>

#include "gemm_device.h"
#include "gemm_instances.h"
#include "launch.h"

namespace sg {

__global__ void k_fill_zero(u4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = u4{0u, 0u, 0u, 0u};
}

__global__ void k_topology(int* out, int n) {
  if (threadIdx.x == 0 && (int)blockIdx.x < n) out[blockIdx.x] = (int)xcc_id();
}

static GemmKernel gemm_kernel(unsigned w_aux, int path, int a, int b) {
  if (w_aux == (unsigned)kAuxNt) return gemm_kernel_nt(path, a, b);
  if (w_aux == 0u) return gemm_kernel_cached(path, a, b);
  if (w_aux == (unsigned)(kAuxNt | kAuxSc1)) return gemm_kernel_sc1(path, a, b);
  return nullptr;
}

bool gemm_variant_exists(int path, int a, int b) { return gemm_kernel_nt(path, a, b) != nullptr; }

hipError_t launch_gemm(const StageDesc& d, int path, int a, int b, int grid, int block, int lds,
                       unsigned* status, hipStream_t stream) {
  GemmKernel k = gemm_kernel(d.w_aux, path, a, b);
  if (!k) return hipErrorInvalidValue;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(block), lds, stream, d, status);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  int grid = (int)((n16 + 255) / 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, stream, (u4*)p, n16);
  return hipGetLastError();
}

hipError_t launch_topology(int* out, int n, hipStream_t stream) {
  hipLaunchKernelGGL(k_topology, dim3(n), dim3(64), 0, stream, out, n);
  return hipGetLastError();
}

}  // namespace sg
