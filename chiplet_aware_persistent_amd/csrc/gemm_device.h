// Device-side building blocks of the small-M decode GEMM on gfx950.
//
// A workgroup executes "items" of a stage: an item is a block of CB = waves*TN
// output columns of its XCD over one K split [s*KS, (s+1)*KS).  Every wave of
// the workgroup owns TN of those columns over the whole split (so no
// reduction between the waves of a workgroup is needed), streams the weight
// rows of its columns from HBM with 16-byte nontemporal buffer loads kept P
// steps ahead in a register ring, reads X from an LDS window that the
// workgroup stages once per split, and accumulates in fp32:
//   * dot2 path (M < 16): the 64 lanes of a wave walk K (8 values each, one
//     contiguous kilobyte of a weight row per load) and v_dot2_f32_bf16 folds
//     pairs into fp32; a reduce-scatter butterfly over the lanes finishes.
//   * MFMA path (M >= 16): v_mfma_f32_16x16x32_bf16 with X as the A operand
//     (from LDS) and W as the B operand (straight from the load registers);
//     every weight fragment feeds all ceil(M/16) m-tiles before it is dropped,
//     which is the M-major reuse of a weight column done in registers.
// MFMA items can also be cut along K inside the workgroup: ksl waves share a
// column group, each streams one K slice, and the slices are added up in slice
// order through LDS at the end of the item (the intra-CTA K-slice of the
// MI355X low-latency GEMM news item, technique 2), which gives every wave a
// share of a small GEMM without going through global memory.
// Item results wait in an LDS stash and are stored after the weight stream:
// vmcnt counts loads and stores in issue order, so a store issued mid-stream
// would make the next wait for a weight load also wait for the store.
// With S > 1 the K splits of a wave tile land in an fp32 workspace and the
// wave that arrives last (arrival counter, old value S-1) adds them up in
// split order and writes Y, so the result does not depend on arrival order.
//
// Weights for XCD x live in the contiguous block of rows [x*Nx, (x+1)*Nx)
// (Fleet reading note, Summary and section 4: Chiplet-task k owns columns
// [k*N/8, (k+1)*N/8) at base + k*(N/8)*K*sizeof(bf16)); the K splits of one
// column block are all processed by workgroups of the same XCD, so partial
// sums never leave that XCD's L2 (section 3b: K-split across XCDs needs fabric
// atomics and is rejected; within an XCD it is the inter-CTA split-K of the
// MI355X low-latency GEMM news item, technique 1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stage_desc.h"

namespace sg {

typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

// Cache-policy bits of gfx950 buffer instructions (aux operand).
constexpr int kAuxSc0 = 1, kAuxNt = 2, kAuxSc1 = 16;

// Status word bits (workspace word 0).
constexpr unsigned kStatusTimeout = 1u;
constexpr unsigned kStatusTopology = 2u;

__device__ __forceinline__ Rsrc make_rsrc(const void* p, unsigned bytes) {
  // 0x00020000: 32-bit data format, the raw-buffer descriptor word 3 of gfx9.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 16-byte loads; an offset at or past the extent returns zeros (buffer range
// check), which is how masked lanes are expressed.
template <int AUX>
__device__ __forceinline__ u4 ld16(Rsrc r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ f4 ld_f4(Rsrc r, unsigned off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}

template <int AUX>
__device__ __forceinline__ void st_f32(Rsrc r, unsigned off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void st_u16(Rsrc r, unsigned off, unsigned short v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void st_f4(Rsrc r, unsigned off, f4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, (int)off, 0, AUX);
}

// fp32 -> bf16 bits, round to nearest even (the hardware conversion of gfx950).
__device__ __forceinline__ unsigned short bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(unsigned short, b);
}

// silu(g) * u in fp32; e^-g as 2^(-g*log2 e) on the hardware exp2.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g / (1.0f + e) * u;
}

// acc + <w, x> over 8 bf16 values, four v_dot2_f32_bf16.  The pairs are
// built from a bf16x8 view: bit-casting the u4 elements one by one (w[i])
// is lowered to four uses of dword 0 by this compiler.
__device__ __forceinline__ float dot8(u4 w, u4 x, float acc) {
  const bf16x8 a = __builtin_bit_cast(bf16x8, w);
  const bf16x8 b = __builtin_bit_cast(bf16x8, x);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {a[2 * i], a[2 * i + 1]};
    const bf16x2 q = {b[2 * i], b[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, q, acc, false);
  }
  return acc;
}

__device__ __forceinline__ void wait_vm0() {
  // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ unsigned xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xF;  // HW_REG_XCC_ID[3:0]
}

// The XCD this workgroup runs on, read from the hardware.  The dispatcher
// hands the workgroups of a launch to the 8 XCDs round-robin, but from a
// starting XCD that changes between launches (graph launches move it), so
// workgroup i runs on XCD (i + r) mod 8 for one r per launch.  Work is indexed
// by (this XCD, i / 8): for a grid of 8 * slots workgroups that covers every
// (XCD, slot) pair once, whatever r is.  An id outside 0..7 (another
// partition mode) is recorded as a topology error.
__device__ __forceinline__ int xcd_of_wg(unsigned* status) {
  const unsigned x = xcc_id();
  if (x >= (unsigned)kXcds && threadIdx.x == 0)
    __hip_atomic_fetch_or(status, kStatusTopology, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (int)(x & 7u);
}

// Placement check of a single launch.  Once its work is done, workgroup (XCD
// x, slot w) sets bit w of the XCD's claim word (control block word
// kClaimWord + x) and looks at the word's old value: a bit that was already
// set means two workgroups ran as the same (XCD, slot) pair, so some other
// pair's columns were never computed, and the topology bit is latched in the
// status word.  Only after its claim has returned does the workgroup count
// itself in the XCD's arrival word (kClaimCount + x); the arrival that
// brings the count to nslots comes after every claim of the XCD in this
// launch, and it clears both words for the next launch.  (Clearing when the
// mask looked complete instead would let a bit set before the launch
// complete the mask early, so that its owner claimed a cleared word.)  A
// broken dispatch leaves some XCD short of nslots arrivals, so its words stay
// set and the error repeats on every later launch until the workspace is
// re-initialised.  The claim goes out after the workgroup's last stores.  Its
// device-scope round trips still end the workgroup 1.5-3 us later on MI355X
// (measured on the M = 1 decode projections), so the check is a plan option
// (SGEMM_F_CHECK_PLACEMENT).
constexpr int kClaimWord = 32;   // byte 128 of the workspace control block
constexpr int kClaimCount = 40;  // byte 160: arrivals per XCD in the current launch

__device__ __forceinline__ void claim_and_check(unsigned* ctl, int xcd, int slot, int nslots) {
  if (threadIdx.x == 0) {
    const unsigned bit = slot < 32 ? 1u << slot : 0u;
    const unsigned old =
        __hip_atomic_fetch_or(ctl + kClaimWord + xcd, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bit == 0u || (old & bit))
      __hip_atomic_fetch_or(ctl, kStatusTopology, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The claim has returned (its value was used above; the wait and the
    // clobber keep the arrival behind it).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const unsigned n =
        __hip_atomic_fetch_add(ctl + kClaimCount + xcd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n + 1u == (unsigned)nslots) {
      __hip_atomic_store(ctl + kClaimWord + xcd, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctl + kClaimCount + xcd, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Reduce-scatter over the 64 lanes of a wave: v holds V (power of two <= 64)
// per-lane partials; afterwards lane l holds the full sum of value l/(64/V).
// Fixed exchange pattern, so the result is bitwise reproducible.  Stage ST
// exchanges over lane distance 32 >> ST; every index is a compile-time
// constant, so v stays in registers.
template <int V, int ST>
__device__ __forceinline__ void reduce_scatter_stage(float (&v)[V], int lane) {
  if constexpr (ST < 6) {
    constexpr int o = 32 >> ST;
    constexpr int half = V >> (ST + 1);
    if constexpr (half >= 1) {
      const bool up = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float send = up ? v[i] : v[i + half];
        const float keep = up ? v[i + half] : v[i];
        v[i] = keep + __shfl_xor(send, o);
      }
    } else {
      v[0] += __shfl_xor(v[0], o);
    }
    reduce_scatter_stage<V, ST + 1>(v, lane);
  }
}

template <int V>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[V], int lane) {
  reduce_scatter_stage<V, 0>(v, lane);
  return v[0];
}

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }

// Split-K arrival.  A wave stores the partial of every (tile, split) it
// computes without waiting; only after its last item does it make the
// partials visible and bump the tile counters, so the weight stream is never
// drained mid-way by a wait on its own stores (vmcnt counts loads and stores
// in issue order).  The wave whose arrival is the S-th (counter old value
// S-1) owns the tile: it resets the counter and adds the S partials in split
// order, so the sum does not depend on which split arrived last.
//   SYNC_XCD: all S contributors run on the same XCD (a tile's counter and
//     partials are indexed by the hardware XCD id), so their partials meet in
//     that XCD's L2.  A contributor's stores go through the write-through
//     vector L1 to the L2; s_waitcnt vmcnt(0) returns once the L2 has
//     acknowledged them, and only then does the counter bump go out.  The
//     owner's bump returns S-1 only after every contributor's bump was
//     performed, and it then reads the partials with sc1 (agent-scope)
//     loads, which miss its own L1 and are served by the same L2.  The
//     workgroup-scope fences emit no instruction on gfx950; they keep the
//     compiler from moving the partial stores below the wait or the owner's
//     loads above its bump.  This is weaker than a device-scope release
//     (an L2 write-back, buffer_wbl2 sc1) and acquire (buffer_inv sc1), which
//     the partials do not need because they never leave the XCD.
//   SYNC_AGENT: device-scope release and acquire, valid whatever the
//     placement.
__device__ __forceinline__ void splitk_release(int sync) {
  if (sync == SYNC_AGENT) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  } else {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vm0();
  }
}

__device__ __forceinline__ unsigned splitk_bump(unsigned* ctr, int lane) {
  unsigned old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

__device__ __forceinline__ bool splitk_own(unsigned* ctr, unsigned old_lane0, int S, int sync, int lane) {
  const unsigned old = __shfl(old_lane0, 0);
  const bool last = old == (unsigned)(S - 1);
  if (last) {
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (sync == SYNC_AGENT) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    } else {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  return last;
}

// Split-K finalize: add the S partials of a tile in split order.  The partial
// loads go out QB splits at a time (S is a run-time value, so a plain loop
// would wait for every split's loads before issuing the next split's).
// Past-S slots read the buffer's extent (zeros) and are not added, so the sum
// is the same sequence of additions as one load per split.
template <int AUX, int QB>
__device__ __forceinline__ float sum_partials(Rsrc pr, unsigned base, unsigned stride, int S, bool valid,
                                              unsigned oob) {
  float t = 0.f;
  for (int q0 = 0; q0 < S; q0 += QB) {
    float p[QB];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      const unsigned off = valid && q0 + qq < S ? (base + (unsigned)(q0 + qq) * stride) * 4u : oob;
      p[qq] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)off, 0, AUX));
    }
#pragma unroll
    for (int qq = 0; qq < QB; ++qq)
      if (q0 + qq < S) t += p[qq];
  }
  return t;
}

template <int AUX, int NT, int MT>
__device__ __forceinline__ void sum_partials_f4(Rsrc pr, unsigned base, unsigned stride, int S, int lane,
                                                f4 (&tot)[NT][MT], unsigned oob) {
  constexpr int QB = 16 / (NT * MT) > 1 ? 16 / (NT * MT) : 1;  // <= 16 fragments in flight
  for (int q0 = 0; q0 < S; q0 += QB) {
    f4 p[QB][NT][MT];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const unsigned e = base + (unsigned)(q0 + qq) * stride + (unsigned)((j * MT + i) * 256 + lane * 4);
          p[qq][j][i] = ld_f4<AUX>(pr, q0 + qq < S ? e * 4u : oob);
        }
#pragma unroll
    for (int qq = 0; qq < QB; ++qq)
      if (q0 + qq < S) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int i = 0; i < MT; ++i) tot[j][i] += p[qq][j][i];
      }
  }
}

// The waves of a workgroup form ng groups of wpi waves; each group is one
// item stream.  Stream q of workgroup slot w runs the contiguous, balanced
// range [i0, i1) of the XCD's items; the ranges of one workgroup's streams
// are adjacent, so their union is contiguous too (one X window serves all).
__device__ __forceinline__ void my_items(int items, int slot, int nslots, int ng, int q, int& i0,
                                         int& i1) {
  const long long nw = (long long)nslots * ng, w = (long long)slot * ng + q;
  i0 = (int)((long long)items * w / nw);
  i1 = (int)((long long)items * (w + 1) / nw);
}

__device__ __forceinline__ int first_item_of_wg(int items, int slot, int nslots) {
  return (int)((long long)items * slot / nslots);
}

// X window: rows [0, rows_p) x columns [k0, k0 + win) of X go to LDS (row
// stride d.xrow elements), zero outside [0,M) x [k0,kend) and in the row
// padding.  The window is filled with gfx950's buffer-to-LDS loads: one wave
// instruction fills one kilobyte of LDS (lane l the 16 bytes at 16 l), and
// each lane fetches the X values that belong at its LDS position, so no
// registers or LDS writes are involved and the loads can be issued ahead of
// the weight ring.  d.red_off (the end of the window region) is a multiple of
// 1 KB, so every chunk stays inside the window region.
__device__ __forceinline__ void stage_x_lds(const StageDesc& d, uint16_t* xs, int rows_p, int k0, int kend,
                                            Rsrc xr) {
  const int lane = threadIdx.x & 63;
  const int nw = (int)(blockDim.x >> 6);
  const int chunks = d.red_off >> 10;
  for (int c = (int)(threadIdx.x >> 6); c < chunks; c += nw) {
    const int e = (c * 1024 + lane * 16) >> 1;  // element of the window buffer
    const int row = e / d.xrow;
    const int col = e - row * d.xrow;
    const int k = k0 + col;
    const bool valid = row < rows_p && row < d.M && col < d.win && k < kend;
    const unsigned off = valid ? ((unsigned)row * (unsigned)d.ldx + (unsigned)k) * 2u : d.x_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)((char*)xs + c * 1024),
                                             16, off, 0, 0, 0);
  }
}

// s_waitcnt vmcnt(n) (n < 64), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Store one output element according to the stage's mode.  Out-of-range
// elements are dropped by the buffer range check (off = extent).
__device__ __forceinline__ void store_out(const StageDesc& d, Rsrc yr, Rsrc y2r, bool ok, int m,
                                          int col, float v) {
  const unsigned e = (unsigned)m * (unsigned)d.ldy + (unsigned)col;
  if (d.R) {  // residual stream: y = x + projection, added in fp32 before the rounding
    const Rsrc rr = make_rsrc(d.R, d.r_bytes);
    const unsigned short x = (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(rr, (int)(ok ? e * 2u : d.r_bytes), 0, 0);
    v += __builtin_bit_cast(float, (unsigned)x << 16);
  }
  if (d.mode == OUT_F32) {
    st_f32<kAuxNt>(yr, ok ? e * 4u : d.y_bytes, v);
  } else {
    st_u16<kAuxNt>(yr, ok ? e * 2u : d.y_bytes, bf16_bits(v));
    if (d.mode == OUT_BF16_F32) st_f32<kAuxNt>(y2r, ok ? e * 4u : d.y2_bytes, v);
  }
}

// ------------------------------------------------------------------ stages
struct NoHook {
  __device__ bool operator()() const { return true; }
};

// Transform of the staged X window, called after the window's loads are
// issued and before they are waited for: it may issue loads of its own, and it
// must leave the window ready (all its loads and its LDS writes complete and
// a workgroup barrier passed).  The default only waits.
struct NoNorm {
  static constexpr bool active = false;
  __device__ void operator()(uint16_t*, int, int, int, int) const {}
};

// Per item: stage X for the item's split (only when it changes), stream the
// item's padded steps through the P-deep ring (the issue cursor runs ahead
// into the next items), reduce, then store Y (S == 1) or the partial.
// pre_x() runs once the first P steps are in flight and before any X is read:
// the chain waits there for the stage producing X.  It is called by every
// workgroup, also one without items.  Returns false if pre_x() did.

// ------------------------------------------------------------------ dot2
// Lane l walks K eight values at a time (one contiguous kilobyte of a weight
// row per 64-lane load); G weight rows per wave share the X registers.
// PAIRED (the chain's gate_up stage): the wave's G rows are G/2 gate rows and
// the G/2 up rows pair_off further on; the wave owns G/2 output columns and
// writes silu(gate) * up.
// Inside the layer chain the round-robin item order is built only for waves
// of at most this many (column, row) sums: with more, its two extra loop
// registers push the chain kernel past the register file.
constexpr int kRrChainMaxMG = 16;

template <int M, int G, int AUX, bool PAIRED = false, typename Hook = NoHook, typename XNorm = NoNorm>
__device__ __forceinline__ bool dot2_stage(const StageDesc& d, uint16_t* xs, int xcd, int slot, int nslots,
                           Hook pre_x = Hook(), XNorm xnorm = XNorm()) {
  constexpr int P = ring_depth_dot2(G);
  constexpr int V = pow2_at_least(G * M);
  static_assert(V <= 64, "G*M must fit one wave");
  static_assert(!PAIRED || G % 2 == 0, "a paired wave holds whole (gate, up) pairs");
  constexpr int GO = PAIRED ? G / 2 : G;  // output columns per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // The stream's items: i0, i0 + istep, ... below i1.  With d.rr (single
  // launches with one K split) stream w of the XCD's nslots * ng takes the
  // items w, w + nslots * ng, ..., so the streams of an XCD read neighbouring
  // weight rows at any one time; otherwise a contiguous balanced range.
  int i0, i1, istep = 1;
  if ((__is_same(Hook, NoHook) || M * G <= kRrChainMaxMG) && d.rr) {
    i0 = slot * d.ng + wave / d.wpi;
    i1 = d.items;
    istep = nslots * d.ng;
  } else {
    my_items(d.items, slot, nslots, d.ng, wave / d.wpi, i0, i1);
  }
  const int nit = i0 < i1 ? (i1 - i0 + istep - 1) / istep : 0;
  const int wv = wave % d.wpi;  // wave's place within its item
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const Rsrc pr = make_rsrc(d.part, d.part_bytes);
  const int spad = d.steps;  // multiple of P
  constexpr int GM = G * M;
  constexpr int grp = 64 / V;
  const int idx = lane / grp;
  const bool owner = (lane % grp) == 0 && idx < GM;
  const int oc = idx / M, om = idx - (idx / M) * M;
  float* stash = (float*)((char*)xs + d.stash_off);  // [wave][stash_cap][64]
  // The finished value of output column oc, row om (lane value r, all lanes
  // call): paired, the up sum of the same column is GO*M values further on.
  auto store_col = [&](int colb, float r) {
    const int col = colb + oc;
    if constexpr (PAIRED) {
      const float u = __shfl(r, lane + GO * M * grp);
      store_out(d, yr, y2r, owner && oc < GO && col < xc1 && om < d.M, om, col, silu_mul(r, u));
    } else {
      store_out(d, yr, y2r, owner && col < xc1 && om < d.M, om, col, r);
    }
  };
  // Result of item `it` (lane value r): Y when S == 1, else the partial.
  auto out_item = [&](int it, float r) {
    const int s = it / d.NB;
    const int b = it - s * d.NB;
    if (d.S == 1) {
      store_col(xc0 + b * d.CB + wv * GO, r);
    } else {
      const unsigned tile = (unsigned)((xcd * d.NB + b) * d.wpi + wv);
      st_f32<0>(pr, owner ? ((tile * d.S + s) * GM + idx) * 4u : d.part_bytes, r);
    }
  };

  u4 ring[P][G];
  // Weight stream.  Slot p of the ring holds step t0+p of the current item;
  // after consuming it the wave issues step t0+P+p, which falls in the next
  // item for the last P steps.  Issue addresses are a per-item base plus a
  // constant stride, and masked lanes (past K, past N, past the last item)
  // point at the end of W, where the buffer range check returns zeros: no
  // branch, so the compiler keeps exact counts of the loads in flight.
  struct Src {
    unsigned base;  // byte offset of (weight row of output column colb, k = k0 + 8*lane)
    int klim;       // steps * kstep with k < kend  -> valid while t*kstep + 8*lane < klim
    int cols;       // output columns of the wave tile that exist (col < xc1)
  };
  auto src_of = [&](int it) -> Src {
    Src r;
    if (it >= i1) { r.base = 0; r.klim = 0; r.cols = 0; return r; }
    const int s_ = it / d.NB;
    const int b_ = it - s_ * d.NB;
    const int k0 = s_ * d.KS;
    const int colb = xc0 + b_ * d.CB + wv * GO;
    r.base = ((unsigned)colb * (unsigned)d.K + (unsigned)k0) * 2u + (unsigned)lane * 16u;
    r.klim = min(d.K, k0 + d.KS) - k0;
    r.cols = min(GO, xc1 - colb);
    return r;
  };
  // Weight row of the wave's row c relative to row colb (paired: up rows
  // pair_off further on).
  auto row_of = [&](int c) -> unsigned {
    return PAIRED && c >= GO ? (unsigned)(d.pair_off + c - GO) : (unsigned)c;
  };
  auto issue = [&](u4(&dst)[G], const Src& sr, int t) {
    const bool kin = t * kDot2KStep + lane * 8 < sr.klim;
#pragma unroll
    for (int c = 0; c < G; ++c) {
      const bool valid = kin && (PAIRED ? c % GO : c) < sr.cols;
      const unsigned off = sr.base + row_of(c) * (unsigned)d.K * 2u + (unsigned)t * (kDot2KStep * 2u);
      dst[c] = ld16<AUX>(wr, valid ? off : d.w_bytes);
    }
  };

  // One X window per workgroup and stage: the K range of every split its
  // items touch (the planner sizes d.win for the widest such range).  In a
  // single launch the window loads go out before the weight ring, so waiting
  // until only the ring's loads are outstanding covers them; in the chain X
  // exists only after the wait, so its loads follow the ring.
  constexpr bool early = __is_same(Hook, NoHook);
  const int s_first = first_item_of_wg(d.items, slot, nslots) / d.NB;
  if constexpr (early) stage_x_lds(d, xs, M, s_first * d.KS, d.K, xr);
  Src sc = src_of(i0), sn = src_of(i0 + istep);
  // Chain: the first q0 steps of the wave's first item are loaded into LDS
  // (buffer-to-LDS, no registers) before the wait for X, so the stage
  // boundary's latency streams weights; the ring then starts at step q0.
  int q0 = 0;
  const uint16_t* wl = nullptr;
  if constexpr (!early) {
    q0 = i0 < i1 ? d.wpf : 0;
    uint16_t* wdst = (uint16_t*)((char*)xs + d.wpf_off) + (size_t)wave * d.wpf * G * 512;
    wl = wdst;
    for (int t = 0; t < q0; ++t) {
      const bool kin = t * kDot2KStep + lane * 8 < sc.klim;
#pragma unroll
      for (int c = 0; c < G; ++c) {
        const bool valid = kin && (PAIRED ? c % GO : c) < sc.cols;
        const unsigned off = sc.base + row_of(c) * (unsigned)d.K * 2u + (unsigned)t * (kDot2KStep * 2u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(wdst + (t * G + c) * 512), 16,
            valid ? off : d.w_bytes, 0, 0, AUX);
      }
    }
  }
  {
    const bool whole = q0 > 0 && q0 == spad;  // the ring starts on the next item
    const Src& rs = whole ? sn : sc;
    const int rt = whole ? 0 : q0;
#pragma unroll
    for (int p = 0; p < P; ++p) issue(ring[p], rs, rt + p);
  }
  if (!pre_x()) return false;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (early) {
    wait_vm<P * G>();
  } else {
    stage_x_lds(d, xs, M, s_first * d.KS, d.K, xr);
    if constexpr (XNorm::active) xnorm(xs, M, d.xrow, s_first * d.KS, d.win);
    wait_vm0();
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  float acc[G][M];
#pragma unroll
  for (int c = 0; c < G; ++c)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[c][m] = 0.f;
  int it = i0, t0 = 0;
  int xoff = (i0 / d.NB - s_first) * d.KS;  // LDS column of the current item's k0
  // Item complete: reduce the lanes' sums, then stash or store the result.
  auto finish_item = [&]() {
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = 0.f;
#pragma unroll
    for (int c = 0; c < G; ++c)
#pragma unroll
      for (int m = 0; m < M; ++m) v[c * M + m] = acc[c][m];
    const float r = wave_reduce_scatter<V>(v, lane);
    const int li = (it - i0) / istep;
    if (li < d.stash_cap) {
      stash[(wave * d.stash_cap + li) * 64 + lane] = r;
    } else {
      out_item(it, r);
    }
#pragma unroll
    for (int c = 0; c < G; ++c)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[c][m] = 0.f;
    it += istep;
    t0 = 0;
    sc = sn;
    sn = src_of(it + istep);
    xoff = (it / d.NB - s_first) * d.KS;
  };
  if constexpr (!early) {
    if (q0 > 0) {  // the first item's LDS steps
      const uint16_t* xb = xs + xoff + lane * 8;
      for (int t = 0; t < q0; ++t) {
        u4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = *(const u4*)(xb + m * d.xrow + t * kDot2KStep);
#pragma unroll
        for (int c = 0; c < G; ++c) {
          const u4 w = *(const u4*)(wl + (t * G + c) * 512 + lane * 8);
#pragma unroll
          for (int m = 0; m < M; ++m) acc[c][m] = dot8(w, xv[m], acc[c][m]);
        }
      }
      t0 = q0;
      if (q0 == spad) finish_item();
    }
  }
  const int total = nit * spad - q0;
  for (int T = 0; T < total; T += P) {
    const bool here = t0 + P < spad;
    const Src& sr = here ? sc : sn;
    const int tn = here ? t0 + P : t0 + P - spad;
    const uint16_t* xb = xs + xoff + t0 * kDot2KStep + lane * 8;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      u4 xv[M];
#pragma unroll
      for (int m = 0; m < M; ++m) xv[m] = *(const u4*)(xb + m * d.xrow + p * kDot2KStep);
#pragma unroll
      for (int c = 0; c < G; ++c)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[c][m] = dot8(ring[p][c], xv[m], acc[c][m]);
      issue(ring[p], sr, tn + p);
      // Pin the reload of slot p right behind its use: otherwise the
      // scheduler sinks all reloads to the end of the unrolled group and the
      // next group has to wait for every load (vmcnt(0)).
      __builtin_amdgcn_sched_barrier(0);
    }
    t0 += P;
    if (t0 == spad) finish_item();
  }

  // Stored items: results of the stream, written after its last load.
  {
    const int n = min(nit, d.stash_cap);
    for (int li = 0; li < n; ++li) out_item(i0 + li * istep, stash[(wave * d.stash_cap + li) * 64 + lane]);
  }

  if (d.S > 1 && i0 < i1) {
    splitk_release(d.sync);
    constexpr int B = 4;  // arrivals in flight at once
    for (int c0 = i0; c0 < i1; c0 += B) {
      unsigned old[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int it = c0 + j;
        const int b = it % d.NB;
        old[j] = it < i1 ? splitk_bump(d.ctr + (xcd * d.NB + b) * d.wpi + wv, lane) : 0u;
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int it = c0 + j;
        if (it >= i1) break;
        const int b = it % d.NB;
        const unsigned tile = (unsigned)((xcd * d.NB + b) * d.wpi + wv);
        if (!splitk_own(d.ctr + tile, old[j], d.S, d.sync, lane)) continue;
        const unsigned base = tile * d.S * GM + idx;
        const float t = d.sync == SYNC_XCD ? sum_partials<kAuxSc1, 8>(pr, base, GM, d.S, owner, d.part_bytes)
                                           : sum_partials<0, 8>(pr, base, GM, d.S, owner, d.part_bytes);
        store_col(xc0 + b * d.CB + wv * GO, t);
      }
    }
  }
  return true;
}

// ------------------------------------------------------------------ MFMA
// NT n-tiles of 16 columns per wave (PAIRED: tile 0 = gate rows, tile 1 = the
// matching up rows pair_off further), MT m-tiles of 16 rows; every weight
// fragment feeds all MT m-tiles.
// Loads read whole 128-byte lines: for a 64-wide k-step of a 16-row n-tile,
// load 0 gives lane l the 16-byte chunk l%8 of row l/8 and load 1 gives it
// chunk (l%8)^4 of row 8 + l/8 (so eight lanes cover one line either way).
// One v_cndmask per dword then gathers the chunks of MFMA half 0 (k 0..31:
// chunks 0-3 of all 16 rows) into one register and those of half 1 into
// another, and one ds_bpermute per dword moves them to the B-operand layout
// (lane l' holds column l'%16 at k-group l'/16).  Issuing each line in one
// instruction halves the L2 requests against two 64-byte halves per line.
// The A operand (X, from LDS) uses the same k slots: for m-tile i lane l'
// reads row 16i + l'%16 (the zero row M where that passes M) at
// k = 32h + 8(l'/16).
template <int MT, int NT, bool PAIRED, int AUX, bool DEEP = false, typename Hook = NoHook, bool MTI = false,
          typename XNorm = NoNorm>
__device__ __forceinline__ bool mfma_stage(const StageDesc& d, uint16_t* xs, int xcd, int slot, int nslots,
                           Hook pre_x = Hook(), XNorm xnorm = XNorm()) {
  constexpr int P = ring_depth_mfma(NT, DEEP);
  constexpr int TW = PAIRED ? 16 : 16 * NT;  // distinct output columns per wave
  constexpr unsigned TILE = NT * MT * 256;   // floats of one wave tile
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  // Items: (split, column block, m-tile), m-tile fastest.  MTI (the m-tile-
  // item variant): d.mtiles items per (split, column block), MT 16-row
  // m-tiles each (a window of 16 MT rows); otherwise one item covers every
  // row.  A stream runs the
  // items i0, i0 + istep, ... below i1: a contiguous range, or with
  // d.interleave every ng-th item of the workgroup's range.
  const int mtl = MTI ? d.mtiles : 1;
  int i0, i1, istep = 1;
  if (MTI && d.interleave) {
    i0 = first_item_of_wg(d.items, slot, nslots) + wave / d.wpi;
    i1 = first_item_of_wg(d.items, slot + 1, nslots);
    istep = d.ng;
  } else if (!MTI && d.rr) {
    // One K split: the items round-robin over the XCD's streams, as in the
    // dot2 path.
    i0 = slot * d.ng + wave / d.wpi;
    i1 = d.items;
    istep = nslots * d.ng;
  } else {
    my_items(d.items, slot, nslots, d.ng, wave / d.wpi, i0, i1);
  }
  const int nit = i0 < i1 ? (i1 - i0 + istep - 1) / istep : 0;  // items of this stream
  // With d.nfast (the M-split order) the column block runs fastest instead:
  // neighbouring items take different weights, so no two m-tiles of a block
  // run at the same time and nothing is shared between them.
  const int per_split = d.NB * mtl;
  const bool nfast = MTI && d.nfast;
  auto split_of = [&](int it) { return it / per_split; };
  auto block_of = [&](int it) {
    const int r = it - split_of(it) * per_split;
    return nfast ? r % d.NB : r / mtl;
  };
  auto mtile_of = [&](int it) {
    if constexpr (!MTI) return 0;
    const int r = it - split_of(it) * per_split;
    return nfast ? r / d.NB : r % mtl;
  };
  const int wv = wave % d.wpi;  // wave's place within its item
  const int CG = d.wpi / d.ksl; // column groups per item
  const int cg = wv % CG;       // this wave's column group
  const int kq = wv / CG;       // this wave's K slice
  const bool owner = kq == 0;   // ends up with the item's tile (then wv == cg)
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const Rsrc pr = make_rsrc(d.part, d.part_bytes);
  const int spad = d.steps;  // multiple of P
  // LDS after the X window: K-slice reduction [CG][ksl-1][NT*MT][64] and the
  // output stash [owner][stash_cap][NT*MT][64], f4 per lane.
  f4* red = (f4*)((char*)xs + d.red_off);
  f4* stash = (f4*)((char*)xs + d.stash_off);
  const int own = d.ksl > 1 ? cg : wave;

  u4 ring[P][NT][2];
  // Weight stream, organised as in the dot2 path (per-item base + constant
  // stride, branch-free masking through the buffer range check).
  struct Src {
    unsigned base;  // byte offset of (weight row of column col0, k = k0)
    int klim;       // chunk c of step t is valid while t*64 + 8c < klim
    int col0;       // first column of n-tile 0 (n-tile j: col0 + 16 j unless paired)
  };
  const int lr8 = lane >> 3;  // row within the 8-row half of the n-tile
  int lch[2];                 // 16-byte chunk this lane loads, per load
  unsigned loff[2];           // its byte offset from the n-tile's (row 0, k0)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lch[h] = (lane & 7) ^ (4 * h);
    loff[h] = ((unsigned)(8 * h + lr8) * (unsigned)d.K + 8u * (unsigned)lch[h]) * 2u;
  }
  auto src_of = [&](int it) -> Src {
    Src r;
    if (it >= i1) { r.base = 0; r.klim = 0; r.col0 = xc1; return r; }
    const int s_ = split_of(it);
    const int b_ = block_of(it);
    const int k0 = s_ * d.KS + kq * d.kss;
    const int col0 = xc0 + b_ * d.CB + cg * TW;
    r.base = ((unsigned)col0 * (unsigned)d.K + (unsigned)k0) * 2u;
    r.klim = min(min(d.K, (s_ + 1) * d.KS) - k0, d.kss);  // <= 0: slice past the split
    r.col0 = col0;
    return r;
  };
  // byte distance between the weight rows of n-tile j and n-tile 0
  const unsigned jstride = PAIRED ? (unsigned)d.pair_off * (unsigned)d.K * 2u : 16u * (unsigned)d.K * 2u;
  auto issue = [&](u4(&dst)[NT][2], const Src& sr, int t) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = sr.col0 + (PAIRED ? 0 : 16 * j) + 8 * h + lr8;
        const bool valid = col < xc1 && t * kMfmaKStep + 8 * lch[h] < sr.klim;
        const unsigned off = sr.base + loff[h] + (unsigned)j * jstride + (unsigned)t * (kMfmaKStep * 2u);
        dst[j][h] = ld16<AUX>(wr, valid ? off : d.w_bytes);
      }
    }
  };
  // Gather: half 0 takes load 0 on lanes with l%8 < 4 and load 1 elsewhere,
  // half 1 the opposite.  Then lane l' = (c = l'%16, g = l'/16) takes the
  // dwords of lane 8(c%8) + 4(c/8 ^ hh) + g (byte address for bpermute).
  const bool lo = (lane & 7) < 4;
  int perm_addr[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) perm_addr[hh] = (8 * (r16 & 7) + 4 * ((r16 >> 3) ^ hh) + g4) * 4;
  auto to_b = [&](const u4(&v)[2], int hh) -> bf16x8 {
    u4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned m = (lo == (hh == 0)) ? v[0][q] : v[1][q];
      o[q] = (unsigned)__builtin_amdgcn_ds_bpermute(perm_addr[hh], (int)m);
    }
    return __builtin_bit_cast(bf16x8, o);
  };

  auto emit = [&](int colb, int j, int i, f4 v, f4 vu) {
    const int col = colb + (PAIRED ? 0 : 16 * j) + r16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * i + 4 * g4 + e;  // i: the m-tile (counted from 0 over all rows)
      const bool ok = m < d.M && col < xc1;
      store_out(d, yr, y2r, ok, m, col, PAIRED ? silu_mul(v[e], vu[e]) : v[e]);
    }
  };
  // The finished tile of item `it` (owner wave): Y when S == 1, else the
  // split's partial.
  auto tile_of = [&](int it) {  // split-K tile (counter and partial block) of item it
    return (unsigned)(((xcd * d.NB + block_of(it)) * d.wpi + wv) * mtl + mtile_of(it));
  };
  auto out_tile = [&](int it, const f4(&v)[NT][MT]) {
    const int s = split_of(it);
    const int b = block_of(it);
    if (d.S == 1) {
      const int colb = xc0 + b * d.CB + wv * TW;
      const int mt = MT * mtile_of(it);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (PAIRED) {
          emit(colb, 0, mt + i, v[0][i], v[1][i]);
        } else {
#pragma unroll
          for (int j = 0; j < NT; ++j) emit(colb, j, mt + i, v[j][i], v[j][i]);
        }
      }
    } else {
      const unsigned tile = tile_of(it);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          st_f4<0>(pr, ((tile * d.S + s) * TILE + (j * MT + i) * 256 + lane * 4) * 4u, v[j][i]);
    }
  };

  // One X window per workgroup and stage: the K range of every split its
  // items touch (the planner sizes d.win for the widest such range).  In a
  // single launch the window loads go out before the weight ring, so waiting
  // until only the ring's loads are outstanding covers them; in the chain X
  // exists only after the wait, so its loads follow the ring.
  constexpr bool early = __is_same(Hook, NoHook);
  const int s_first = split_of(first_item_of_wg(d.items, slot, nslots));
  // The window holds rows [0, M) and, when the M-tiles overhang M, one zero
  // row (row M) that the overhanging lanes of the A operand read instead.
  const int xrows = min(16 * MT * mtl, d.M + 1);
  int xro[MT];
  auto set_rows = [&](int it) {  // A-operand row offsets of item it's m-tiles
    const int m0 = 16 * MT * (it < i1 ? mtile_of(it) : 0);
#pragma unroll
    for (int i = 0; i < MT; ++i) xro[i] = min(m0 + 16 * i + r16, d.M) * d.xrow;
  };
  set_rows(i0);
  if constexpr (early) stage_x_lds(d, xs, xrows, s_first * d.KS, d.K, xr);
  Src sc = src_of(i0), sn = src_of(i0 + istep);
#pragma unroll
  for (int p = 0; p < P; ++p) issue(ring[p], sc, p);
  if (!pre_x()) return false;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (early) {
    wait_vm<P * NT * 2>();
  } else {
    stage_x_lds(d, xs, xrows, s_first * d.KS, d.K, xr);
    if constexpr (XNorm::active) xnorm(xs, d.M, d.xrow, s_first * d.KS, d.win);
    wait_vm0();
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  f4 acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = f4{0.f, 0.f, 0.f, 0.f};
  int it = i0, li = 0, t0 = 0;
  int xoff = (split_of(i0) - s_first) * d.KS + kq * d.kss;
  const int total = nit * spad;
  for (int T = 0; T < total; T += P) {
    const bool here = t0 + P < spad;
    const Src& sr = here ? sc : sn;
    const int tn = here ? t0 + P : t0 + P - spad;
    const uint16_t* xb0 = xs + xoff + t0 * kMfmaKStep + 8 * g4;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint16_t* xb = xb0 + p * kMfmaKStep;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 xa[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
          xa[i] = __builtin_bit_cast(bf16x8, *(const u4*)(xb + xro[i] + 32 * h));
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const bf16x8 wb = to_b(ring[p][j], h);
#pragma unroll
          for (int i = 0; i < MT; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], wb, acc[j][i], 0, 0, 0);
        }
      }
      issue(ring[p], sr, tn + p);
      __builtin_amdgcn_sched_barrier(0);  // as in the dot2 path
    }
    t0 += P;
    if (t0 == spad) {  // item complete
      if (d.ksl > 1) {
        // Slices 1..ksl-1 hand their sums to the slice-0 wave, which adds
        // them in slice order.  All waves of the workgroup share one item
        // stream here, so they reach these barriers together.
        if (!owner) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i)
              red[((cg * (d.ksl - 1) + kq - 1) * (NT * MT) + j * MT + i) * 64 + lane] = acc[j][i];
        }
        __syncthreads();
        if (owner) {
          for (int q = 1; q < d.ksl; ++q) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
              for (int i = 0; i < MT; ++i)
                acc[j][i] += red[((cg * (d.ksl - 1) + q - 1) * (NT * MT) + j * MT + i) * 64 + lane];
          }
        }
        __syncthreads();
      }
      if (owner) {
        if (li < d.stash_cap) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i) stash[((own * d.stash_cap + li) * (NT * MT) + j * MT + i) * 64 + lane] = acc[j][i];
        } else {
          // Stash full (the planner allows this only with S > 1): the
          // split's partial goes out now.  Only this plain store sits in the
          // loop, which keeps the epilogue's registers out of it.
          const int s = split_of(it);
          const unsigned tile = tile_of(it);
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i)
              st_f4<0>(pr, ((tile * d.S + s) * TILE + (j * MT + i) * 256 + lane * 4) * 4u, acc[j][i]);
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[j][i] = f4{0.f, 0.f, 0.f, 0.f};
      it += istep;
      ++li;
      t0 = 0;
      sc = sn;
      sn = src_of(it + istep);
      xoff = (split_of(it) - s_first) * d.KS + kq * d.kss;
      if constexpr (MTI) set_rows(it);
    }
  }

  // Stored items: results of the stream, written after its last load.
  if (owner) {
    const int n = min(nit, d.stash_cap);
    for (int li = 0; li < n; ++li) {
      f4 v[NT][MT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) v[j][i] = stash[((own * d.stash_cap + li) * (NT * MT) + j * MT + i) * 64 + lane];
      out_tile(i0 + li * istep, v);
    }
  }

  if (d.S > 1 && i0 < i1 && owner) {
    splitk_release(d.sync);
    constexpr int B = 4;
    for (int c0 = 0; c0 < nit; c0 += B) {
      unsigned old[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int it = i0 + (c0 + j) * istep;
        old[j] = c0 + j < nit ? splitk_bump(d.ctr + tile_of(it), lane) : 0u;
      }
#pragma unroll
      for (int jj = 0; jj < B; ++jj) {
        const int it = i0 + (c0 + jj) * istep;
        if (c0 + jj >= nit) break;
        const int b = block_of(it);
        const unsigned tile = tile_of(it);
        if (!splitk_own(d.ctr + tile, old[jj], d.S, d.sync, lane)) continue;
        f4 tot[NT][MT];
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int i = 0; i < MT; ++i) tot[j][i] = f4{0.f, 0.f, 0.f, 0.f};
        if (d.sync == SYNC_XCD) {
          sum_partials_f4<kAuxSc1, NT, MT>(pr, tile * d.S * TILE, TILE, d.S, lane, tot, d.part_bytes);
        } else {
          sum_partials_f4<0, NT, MT>(pr, tile * d.S * TILE, TILE, d.S, lane, tot, d.part_bytes);
        }
        const int colb = xc0 + b * d.CB + wv * TW;
        const int mt = MT * mtile_of(it);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (PAIRED) {
            emit(colb, 0, mt + i, tot[0][i], tot[1][i]);
          } else {
#pragma unroll
            for (int j = 0; j < NT; ++j) emit(colb, j, mt + i, tot[j][i], tot[j][i]);
          }
        }
      }
    }
  }
  return true;
}

}  // namespace sg
