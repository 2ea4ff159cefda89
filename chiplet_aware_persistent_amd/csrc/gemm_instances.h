// Instantiation of the single-GEMM kernels for one weight cache policy.
// Each gemm_<policy>.hip includes this with SG_AUX and SG_NAME defined, so
// the three policies compile in parallel translation units.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_device.h"
#include "kc_device.h"

namespace sg {

typedef void (*GemmKernel)(StageDesc, unsigned*);

// ctl: the workspace control block (word 0 status, claim words at kClaimWord).
template <int M, int G, int AUX>
__global__ __launch_bounds__(512) void k_gemm_dot2(StageDesc d, unsigned* ctl) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int xcd = xcd_of_wg(ctl), slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  dot2_stage<M, G, AUX>(d, lds, xcd, slot, nslots);
  if (d.check) claim_and_check(ctl, xcd, slot, nslots);
}

template <int MT, int NT, int AUX, bool MTI = false>
__global__ __launch_bounds__(512) void k_gemm_mfma(StageDesc d, unsigned* ctl) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int xcd = xcd_of_wg(ctl), slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  mfma_stage<MT, NT, false, AUX, false, NoHook, MTI>(d, lds, xcd, slot, nslots);
  if (d.check) claim_and_check(ctl, xcd, slot, nslots);
}

template <int MT, int NTW, int AUX>
__global__ __launch_bounds__(512) void k_gemm_kc(StageDesc d, unsigned* ctl) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int xcd = xcd_of_wg(ctl), slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  mfma_kc_stage<MT, NTW, false, AUX>(d, lds, xcd, slot, nslots);
  if (d.check) claim_and_check(ctl, xcd, slot, nslots);
}

// K-chunked MFMA path (path 3): MT = 1..4 m-tiles, NTW = 2, 3, 4, 6 or 8 tiles per
// item (8 only up to two m-tiles: its accumulators and loads would not fit
// the registers next to four).  Weights nt only.
inline bool kc_variant_ok(int mt, int ntw) {
  return mt >= 1 && mt <= 4 && (ntw == 2 || ntw == 3 || ntw == 4 || ntw == 6 || (ntw == 8 && mt <= 2));
}

template <int AUX>
GemmKernel gemm_kernel_kc(int a, int b) {
  if constexpr (AUX != kAuxNt) {
    return nullptr;
  } else {
#define SG_KC(mt)                                               \
  case mt:                                                      \
    if (b == 2) return k_gemm_kc<mt, 2, AUX>;                   \
    if (b == 3) return k_gemm_kc<mt, 3, AUX>;                   \
    if (b == 4) return k_gemm_kc<mt, 4, AUX>;                   \
    if (b == 6) return k_gemm_kc<mt, 6, AUX>;                   \
    if (b == 8 && mt <= 2) return k_gemm_kc<(mt <= 2 ? mt : 2), 8, AUX>; \
    return nullptr;
    switch (a) {
      SG_KC(1) SG_KC(2) SG_KC(3) SG_KC(4)
      default: return nullptr;
    }
#undef SG_KC
  }
}

// Large-tile MFMA path (gemm_lt.hip): path 5 four waves, path 6 eight;
// weights nt or, cached, with the default policy.
GemmKernel gemm_kernel_lt(int waves, int a, int b, bool cached);

// dot2: M = 1..15, G in {1, 2, 3, 4, 8} with G*M <= 64.  MFMA: MT = 1..4, NT = 1, 2.
// Path 2: the MFMA m-tile-item variant (MT = 1, 2 with NT = 1, 2; MT = 4 with NT = 1).
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
  if (path == 3) return gemm_kernel_kc<AUX>(a, b);
  if (path == 5 || path == 6) {
    if (AUX != kAuxNt && AUX != 0) return nullptr;
    return gemm_kernel_lt(path == 6 ? 8 : 4, a, b, AUX == 0);
  }
  if (path == 2) {  // m-tile items with a window of 16, 32 or 64 rows
    if (a == 1) return b == 1 ? k_gemm_mfma<1, 1, AUX, true> : (b == 2 ? k_gemm_mfma<1, 2, AUX, true> : nullptr);
    if (a == 2) return b == 1 ? k_gemm_mfma<2, 1, AUX, true> : (b == 2 ? k_gemm_mfma<2, 2, AUX, true> : nullptr);
    if (a == 4) return b == 1 ? k_gemm_mfma<4, 1, AUX, true> : nullptr;
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
