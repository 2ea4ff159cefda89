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

// Streaming read of n16 16-byte chunks with nontemporal buffer loads, eight
// in flight per lane.  Every dword is xor-folded and each workgroup xors its
// fold into *sink, so a host-side xor of the buffer checks that every byte was
// read exactly once.  The attainable-bandwidth reference for the weight
// stream.
//   PATTERN 0: grid-stride; consecutive lanes and workgroups read consecutive
//              chunks.
//   PATTERN 1: XCD x (workgroup i on XCD i % 8) reads the x-th eighth of the
//              buffer, each wave a contiguous share of it in 1 KB units, as
//              the decode GEMM reads its per-XCD weight slices.
__device__ __forceinline__ unsigned fold(u4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <int PATTERN>
__global__ __launch_bounds__(512) void k_stream_read(const void* src, unsigned n16, unsigned* sink) {
  const Rsrc r = make_rsrc(src, n16 * 16u);
  const unsigned lane = threadIdx.x & 63;
  unsigned acc = 0;
  if constexpr (PATTERN == 0) {
    const unsigned nth = gridDim.x * blockDim.x;
    unsigned i = blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 7u * nth < n16; i += 8u * nth) {
      u4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld16<kAuxNt>(r, (i + (unsigned)u * nth) * 16u);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += nth) acc ^= fold(ld16<kAuxNt>(r, i * 16u));
  } else {
    const unsigned wpb = blockDim.x >> 6;
    const unsigned xcd = xcc_id() & 7u, slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
    const unsigned units = n16 >> 6;  // whole kilobytes
    const unsigned u0 = (unsigned)((unsigned long long)units * xcd / 8);
    const unsigned u1 = (unsigned)((unsigned long long)units * (xcd + 1) / 8);
    const unsigned long long nw = (unsigned long long)nslots * wpb, w = (unsigned long long)slot * wpb + (threadIdx.x >> 6);
    const unsigned a0 = u0 + (unsigned)((u1 - u0) * w / nw), a1 = u0 + (unsigned)((u1 - u0) * (w + 1) / nw);
    for (unsigned a = a0; a < a1; a += 8) {
      u4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld16<kAuxNt>(r, a + u < a1 ? ((a + u) * 64u + lane) * 16u : n16 * 16u);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= fold(v[u]);
    }
    if (blockIdx.x == gridDim.x - 1 && (threadIdx.x >> 6) == wpb - 1)  // chunks past the last whole kilobyte
      for (unsigned i = units * 64u + lane; i < n16; i += 64u) acc ^= fold(ld16<kAuxNt>(r, i * 16u));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (unsigned)__shfl_xor((int)acc, o);
  __shared__ unsigned part[kMaxWaves];
  if (lane == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
    for (unsigned i = 0; i < (blockDim.x >> 6); ++i) t ^= part[i];
    __hip_atomic_fetch_xor(sink, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_stream_read(const void* src, size_t bytes, int pattern, unsigned* sink, int grid,
                              hipStream_t stream) {
  const unsigned n16 = (unsigned)(bytes / 16);
  if (pattern == 0) {
    hipLaunchKernelGGL(k_stream_read<0>, dim3(grid), dim3(512), 0, stream, src, n16, sink);
  } else {
    hipLaunchKernelGGL(k_stream_read<1>, dim3(grid), dim3(512), 0, stream, src, n16, sink);
  }
  return hipGetLastError();
}

hipError_t launch_topology(int* out, int n, hipStream_t stream) {
  hipLaunchKernelGGL(k_topology, dim3(n), dim3(64), 0, stream, out, n);
  return hipGetLastError();
}

}  // namespace sg
