// Large-tile MFMA kernels of the single GEMM (lt_device.h), weights nt.
// Four waves of one workgroup per CU, so each wave may hold the register file
// of a whole SIMD (accumulators in the accumulation registers).
#include "gemm_instances.h"
#include "lt_device.h"

namespace sg {

template <int MW, int NW, int AUX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_lt(StageDesc d,
                                                                                              unsigned* ctl) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int xcd = xcd_of_wg(ctl), slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  lt_stage<MW, NW, 4, AUX>(d, lds, xcd, slot, nslots);
  if (d.check) claim_and_check(ctl, xcd, slot, nslots);
}

// Eight waves, two per SIMD: each keeps at most half a SIMD's registers.
template <int MW, int NW, int AUX>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_lt8(StageDesc d,
                                                                                               unsigned* ctl) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int xcd = xcd_of_wg(ctl), slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  lt_stage<MW, NW, 8, AUX>(d, lds, xcd, slot, nslots);
  if (d.check) claim_and_check(ctl, xcd, slot, nslots);
}

template <int AUX>
static GemmKernel lt_kernel(int waves, int a, int b) {
  if (waves == 4) {
    if (a == 2 && b == 3) return k_gemm_lt<2, 3, AUX>;
    if (a == 4 && b == 3) return k_gemm_lt<4, 3, AUX>;
    if (a == 4 && b == 6) return k_gemm_lt<4, 6, AUX>;
    if (a == 8 && b == 3) return k_gemm_lt<8, 3, AUX>;
  } else if (waves == 8) {
    if (a == 2 && b == 3) return k_gemm_lt8<2, 3, AUX>;
    if (a == 4 && b == 3) return k_gemm_lt8<4, 3, AUX>;
    if (a == 4 && b == 6) return k_gemm_lt8<4, 6, AUX>;
    if (a == 8 && b == 3) return k_gemm_lt8<8, 3, AUX>;
  }
  return nullptr;
}

// (MW, NW): MW x NW 16 x 16 tiles per wave; the workgroup tile is 32 MW rows
// by 32 NW (four waves, path 5) or 64 NW (eight waves, path 6) columns.
// Weights nt, or with the default cache policy (cached = true).
GemmKernel gemm_kernel_lt(int waves, int a, int b, bool cached) {
  return cached ? lt_kernel<0>(waves, a, b) : lt_kernel<kAuxNt>(waves, a, b);
}

}  // namespace sg
