// Single-GEMM kernels of the decode GEMM (one launch per sgemm_run), the
// workspace fill kernel and the XCD topology probe.
#include <hip/hip_runtime.h>

#include "gemm_device.h"
#include "launch.h"

namespace sg {

constexpr int kRing = 2;  // weight k-steps kept in flight per wave

template <int M, int G>
__global__ __launch_bounds__(512) void k_gemm_dot2(StageDesc d, unsigned* status) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  check_topology(status);
  dot2_stage<M, G, kRing>(d, lds, blockIdx.x & 7, blockIdx.x >> 3, gridDim.x >> 3);
}

template <int MT, int NT>
__global__ __launch_bounds__(512) void k_gemm_mfma(StageDesc d, unsigned* status) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  check_topology(status);
  mfma_stage<MT, NT, kRing, false>(d, lds, blockIdx.x & 7, blockIdx.x >> 3, gridDim.x >> 3);
}

__global__ void k_fill_zero(u4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = u4{0u, 0u, 0u, 0u};
}

__global__ void k_topology(int* out, int n) {
  if (threadIdx.x == 0 && (int)blockIdx.x < n) out[blockIdx.x] = (int)xcc_id();
}

typedef void (*GemmKernel)(StageDesc, unsigned*);

// dot2 instantiations: M = 1..15, G in {4, 8} with G*M <= 64.
template <int M>
static GemmKernel dot2_for_g(int g) {
  if (g == 4) return k_gemm_dot2<M, 4>;
  if (g == 8 && M * 8 <= 64) return k_gemm_dot2<M, (M * 8 <= 64 ? 8 : 4)>;
  return nullptr;
}

static GemmKernel dot2_kernel(int m, int g) {
  switch (m) {
    case 1: return dot2_for_g<1>(g);
    case 2: return dot2_for_g<2>(g);
    case 3: return dot2_for_g<3>(g);
    case 4: return dot2_for_g<4>(g);
    case 5: return dot2_for_g<5>(g);
    case 6: return dot2_for_g<6>(g);
    case 7: return dot2_for_g<7>(g);
    case 8: return dot2_for_g<8>(g);
    case 9: return dot2_for_g<9>(g);
    case 10: return dot2_for_g<10>(g);
    case 11: return dot2_for_g<11>(g);
    case 12: return dot2_for_g<12>(g);
    case 13: return dot2_for_g<13>(g);
    case 14: return dot2_for_g<14>(g);
    case 15: return dot2_for_g<15>(g);
    default: return nullptr;
  }
}

template <int MT>
static GemmKernel mfma_for_nt(int nt) {
  if (nt == 1) return k_gemm_mfma<MT, 1>;
  if (nt == 2) return k_gemm_mfma<MT, 2>;
  return nullptr;
}

static GemmKernel mfma_kernel(int mt, int nt) {
  switch (mt) {
    case 1: return mfma_for_nt<1>(nt);
    case 2: return mfma_for_nt<2>(nt);
    case 3: return mfma_for_nt<3>(nt);
    case 4: return mfma_for_nt<4>(nt);
    default: return nullptr;
  }
}

bool gemm_variant_exists(int path, int a, int b) {
  return (path == 0 ? dot2_kernel(a, b) : mfma_kernel(a, b)) != nullptr;
}

hipError_t launch_gemm(const StageDesc& d, int path, int a, int b, int grid, int block, int lds,
                       unsigned* status, hipStream_t stream) {
  GemmKernel k = path == 0 ? dot2_kernel(a, b) : mfma_kernel(a, b);
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
