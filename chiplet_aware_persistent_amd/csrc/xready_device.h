// Chain stages that start on their own XCD's slice of X.
//
// A stage's X is the previous stage's output, and XCD x produced its columns
// [x Nx_p, (x+1) Nx_p): this stage's K values in that range (Fleet reading
// note, section 4 runtime layout: XCD k owns columns [k N/8, (k+1) N/8) of
// every projection).  Those values are in XCD x's own L2 as soon as its
// workgroups have finished (each waited for its stores before its bump of
// the XCD counter, section 2 flowchart (b)), well before the XCD's write-back
// and the global counter that make the other seven slices readable.  So a
// workgroup runs
//   phase 1: for every item of its waves, the K steps of its own XCD's slice,
//            once its XCD's counter is complete;
//   phase 2: the other seven slices, after the global event (acquire).
// Phase 1's per-lane sums wait in LDS.  An item's sum is its own-slice steps
// in order, then the remaining steps in ascending K: fixed per output column,
// so results are bitwise repeatable.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_device.h"

namespace sg {

// X window restricted to K values [kb, ke) (S == 1 window: LDS column = k).
// Every window chunk is issued; lanes outside the range load zeros (the
// window is restaged whole in phase 2).  AUXX: cache bits of the loads.
template <int AUXX>
__device__ __forceinline__ void stage_x_lds_range(const StageDesc& d, uint16_t* xs, int rows_p, int kb, int ke,
                                                  Rsrc xr) {
  const int lane = threadIdx.x & 63;
  const int nw = (int)(blockDim.x >> 6);
  const int chunks = d.red_off >> 10;
  for (int c = (int)(threadIdx.x >> 6); c < chunks; c += nw) {
    const int e = (c * 1024 + lane * 16) >> 1;
    const int row = e / d.xrow;
    const int k = e - row * d.xrow;
    const bool valid = row < rows_p && row < d.M && k < d.win && k >= kb && k < ke && k < d.K;
    const unsigned off = valid ? ((unsigned)row * (unsigned)d.ldx + (unsigned)k) * 2u : d.x_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)((char*)xs + c * 1024),
                                             16, off, 0, 0, AUXX);
  }
}

// dot2 stage, own slice first.  Requires (checked by the planner): S == 1,
// one wave per item stream (wpi == 1), K a whole number of 512-wide steps and
// exactly eight slices of d.own_steps steps, at most d.own_cap items per
// stream.  wait_local() waits for the own XCD's producers, wait_global() for
// the whole previous event (with its acquire); both are workgroup-wide.
template <int M, int G, int AUX, bool PAIRED, typename WaitLocal, typename WaitGlobal>
__device__ __forceinline__ bool dot2_stage_own_first(const StageDesc& d, uint16_t* xs, int xcd, int slot,
                                                     int nslots, WaitLocal wait_local, WaitGlobal wait_global) {
  constexpr int P = ring_depth_dot2(G);
  constexpr int V = pow2_at_least(G * M);
  static_assert(V <= 64, "G*M must fit one wave");
  static_assert(!PAIRED || G % 2 == 0, "a paired wave holds whole (gate, up) pairs");
  constexpr int GO = PAIRED ? G / 2 : G;
  constexpr int GM = G * M;
  constexpr int grp = 64 / V;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int i0, i1;
  my_items(d.items, slot, nslots, d.ng, wave, i0, i1);
  const int n = i1 - i0;
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const int steps = d.K / kDot2KStep;
  const int spx = d.own_steps;
  const int o0 = xcd * spx, o1 = o0 + spx;  // own steps [o0, o1)
  const int first2 = o0 == 0 ? o1 : 0;      // phase 2: first and last step of an item
  const int last2 = o1 == steps ? o0 - 1 : steps - 1;
  const int idx = lane / grp;
  const bool owner = (lane % grp) == 0 && idx < GM;
  const int oc = idx / M, om = idx - (idx / M) * M;
  float* part1 = (float*)((char*)xs + d.own_off) + (size_t)wave * d.own_cap * GM * 64;

  // Cursor over the wave's step sequence: phase 1 visits steps [o0, o1) of
  // items 0..n-1, phase 2 the other steps of items 0..n-1.  Past the end
  // (phase 2, li == n) it stays on a valid step of no item.
  struct Cur {
    int ph, li, t;
  };
  auto start = [&]() -> Cur {
    Cur c;
    c.ph = n > 0 ? 0 : 1;
    c.li = 0;
    c.t = n > 0 ? o0 : first2;
    return c;
  };
  auto advance = [&](Cur& c) {
    if (c.ph == 0) {
      if (++c.t == o1) {
        c.t = o0;
        if (++c.li == n) { c.ph = 1; c.li = 0; c.t = first2; }
      }
    } else if (c.li < n) {
      ++c.t;
      if (c.t == o0) c.t = o1;
      if (c.t >= steps) { c.t = first2; ++c.li; }
    }
  };
  auto row_of = [&](int c) -> unsigned {
    return PAIRED && c >= GO ? (unsigned)(d.pair_off + c - GO) : (unsigned)c;
  };
  auto issue = [&](u4(&dst)[G], const Cur& c) {
    const int colb = xc0 + (i0 + c.li) * d.CB;
    const int cols = c.li < n ? min(GO, xc1 - colb) : 0;
    const unsigned base = ((unsigned)colb * (unsigned)d.K + (unsigned)c.t * kDot2KStep) * 2u + (unsigned)lane * 16u;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const bool valid = (PAIRED ? j % GO : j) < cols;
      dst[j] = ld16<AUX>(wr, valid ? base + row_of(j) * (unsigned)d.K * 2u : d.w_bytes);
    }
  };
  auto store_col = [&](int colb, float r) {
    const int col = colb + oc;
    if constexpr (PAIRED) {
      const float u = __shfl(r, lane + GO * M * grp);
      store_out(d, yr, y2r, owner && oc < GO && col < xc1 && om < d.M, om, col, silu_mul(r, u));
    } else {
      store_out(d, yr, y2r, owner && col < xc1 && om < d.M, om, col, r);
    }
  };

  u4 ring[P][G];
  Cur ic = start();
#pragma unroll
  for (int p = 0; p < P; ++p) {
    issue(ring[p], ic);
    advance(ic);
  }
  if (!wait_local()) return false;
  __builtin_amdgcn_sched_barrier(0);
  // The own slice was written by this XCD's workgroups: it is in this XCD's
  // L2, and sc1 loads do not take it from the CU's L1.
  stage_x_lds_range<kAuxSc1>(d, xs, M, o0 * kDot2KStep, o1 * kDot2KStep, xr);
  wait_vm0();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // Phase 2 entry (every wave once): the other slices after the global event.
  bool in2 = false;
  auto enter2 = [&]() -> bool {
    if (!wait_global()) return false;
    stage_x_lds_range<0>(d, xs, M, 0, d.K, xr);
    wait_vm0();
    __syncthreads();
    return true;
  };

  float acc[G][M];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[j][m] = 0.f;
  Cur cc = start();
  const int total = n * steps;
  for (int u = 0; u < total; u += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (cc.ph == 1 && !in2) {
        if (!enter2()) return false;
        in2 = true;
      }
      if (cc.ph == 1 && cc.t == first2 && cc.li < n) {  // phase-2 start of an item: its own-slice sum
        const float* src = part1 + (size_t)cc.li * GM * 64 + lane;
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[j][m] = src[(j * M + m) * 64];
      }
      const uint16_t* xb = xs + cc.t * kDot2KStep + lane * 8;
      u4 xv[M];
#pragma unroll
      for (int m = 0; m < M; ++m) xv[m] = *(const u4*)(xb + m * d.xrow);
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = dot8(ring[p][j], xv[m], acc[j][m]);
      issue(ring[p], ic);
      advance(ic);
      __builtin_amdgcn_sched_barrier(0);
      if (cc.ph == 0 && cc.t == o1 - 1) {  // phase-1 end of an item: park its sum
        float* dst = part1 + (size_t)cc.li * GM * 64 + lane;
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int m = 0; m < M; ++m) {
            dst[(j * M + m) * 64] = acc[j][m];
            acc[j][m] = 0.f;
          }
      } else if (cc.ph == 1 && cc.t == last2 && cc.li < n) {  // item complete
        float v[V];
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int m = 0; m < M; ++m) {
            v[j * M + m] = acc[j][m];
            acc[j][m] = 0.f;
          }
        const float r = wave_reduce_scatter<V>(v, lane);
        store_col(xc0 + (i0 + cc.li) * d.CB, r);
      }
      advance(cc);
    }
  }
  if (!in2 && !enter2()) return false;
  return true;
}

}  // namespace sg
