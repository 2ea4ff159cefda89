// Instantiation of the single-GEMM kernels for one weight cache policy.
// Each gemm_<policy>.hip includes this with SG_AUX and SG_NAME defined, so
// the three policies compile in parallel translation units.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_device.h"

namespace sg {

typedef void (*GemmKernel)(StageDesc, unsigned*);

template <int M, int G, int AUX>
__global__ __launch_bounds__(512) void k_gemm_dot2(StageDesc d, unsigned* status) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  dot2_stage<M, G, AUX>(d, lds, xcd_of_wg(status), blockIdx.x >> 3, gridDim.x >> 3);
}

template <int MT, int NT, int AUX, bool MTI = false>
__global__ __launch_bounds__(512) void k_gemm_mfma(StageDesc d, unsigned* status) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  mfma_stage<MT, NT, false, AUX, false, NoHook, MTI>(d, lds, xcd_of_wg(status), blockIdx.x >> 3, gridDim.x >> 3);
}

// dot2: M = 1..15, G in {1, 2, 3, 4, 8} with G*M <= 64.  MFMA: MT = 1..4, NT = 1, 2.
// Path 2: the MFMA m-tile-item variant (MT = 1, NT = 1, 2).
template <int AUX>
GemmKernel gemm_kernel_for(int path, int a, int b) {
#define SG_D2(m)                                                    \
  case m:                                                           \
    if (b == 1) return k_gemm_dot2<m, 1, AUX>;                      \
    if (b == 2) return k_gemm_dot2<m, 2, AUX>;                      \
    if (b == 3) return k_gemm_dot2<m, 3, AUX>;                      \
    if (b == 4) return k_gemm_dot2<m, 4, AUX>;                      \
    if (b == 8 && m * 8 <= 64) return k_gemm_dot2<m, (m * 8 <= 64 ? 8 : 4), AUX>; \
    return nullptr;
#define SG_MF(mt)                                   \
  case mt:                                          \
    if (b == 1) return k_gemm_mfma<mt, 1, AUX>;     \
    if (b == 2) return k_gemm_mfma<mt, 2, AUX>;     \
    return nullptr;
  if (path == 2) {
    if (a != 1) return nullptr;
    if (b == 1) return k_gemm_mfma<1, 1, AUX, true>;
    if (b == 2) return k_gemm_mfma<1, 2, AUX, true>;
    return nullptr;
  }
  if (path == 0) {
    switch (a) {
      SG_D2(1) SG_D2(2) SG_D2(3) SG_D2(4) SG_D2(5) SG_D2(6) SG_D2(7) SG_D2(8)
      SG_D2(9) SG_D2(10) SG_D2(11) SG_D2(12) SG_D2(13) SG_D2(14) SG_D2(15)
      default: return nullptr;
    }
  }
  switch (a) {
    SG_MF(1) SG_MF(2) SG_MF(3) SG_MF(4)
    default: return nullptr;
  }
#undef SG_D2
#undef SG_MF
}

GemmKernel gemm_kernel_nt(int path, int a, int b);      // weights nt
GemmKernel gemm_kernel_cached(int path, int a, int b);  // weights default policy
GemmKernel gemm_kernel_sc1(int path, int a, int b);     // weights sc1|nt

}  // namespace sg
