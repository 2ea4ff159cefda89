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

__device__ __forceinline__ u4 ld16_pol(Rsrc r, unsigned off, unsigned aux) {
  if (aux == kAuxNt) return ld16<kAuxNt>(r, off);
  if (aux == (kAuxNt | kAuxSc1)) return ld16<kAuxNt | kAuxSc1>(r, off);
  return ld16<0>(r, off);
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

// Record (once per workgroup) that this workgroup did not run on the XCD its
// index assigns it to under round-robin dispatch.
__device__ __forceinline__ void check_topology(unsigned* status) {
  if (threadIdx.x == 0 && xcc_id() != (blockIdx.x & 7u))
    __hip_atomic_fetch_or(status, kStatusTopology, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reduce-scatter over the 64 lanes of a wave: v holds V (power of two <= 64)
// per-lane partials; afterwards lane l holds the full sum of value l/(64/V).
// Fixed exchange pattern, so the result is bitwise reproducible.
template <int V>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[V], int lane) {
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int o = 32 >> st;
    const int half = V >> (st + 1);
    const bool up = (lane & o) != 0;
    if (half >= 1) {
#pragma unroll
      for (int i = 0; i < (half > 0 ? half : 1); ++i) {
        const float send = up ? v[i] : v[i + half];
        const float keep = up ? v[i + half] : v[i];
        v[i] = keep + __shfl_xor(send, o);
      }
    } else {
      v[0] += __shfl_xor(v[0], o);
    }
  }
  return v[0];
}

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }

// Split-K arrival of one wave tile.  The wave's partial stores are issued
// before the call.  Returns true on the wave that completes the tile (its
// arrival is the S-th); that wave then owns the reduction and has reset the
// counter for the next use.
//   SYNC_XCD: all S contributors run on the same XCD, so their partials meet
//     in one L2: wait until our stores are acknowledged (vmcnt), bump the
//     counter; the reader bypasses its L1 (sc1 loads).
//   SYNC_AGENT: device-scope release (L2 write-back) and acquire (L1/L2
//     invalidate), valid whatever the placement.
__device__ __forceinline__ bool wave_arrive(unsigned* ctr, int S, int sync, int lane) {
  if (sync == SYNC_AGENT) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  } else {
    wait_vm0();
  }
  unsigned old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  const bool last = old == (unsigned)(S - 1);
  if (last) {
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (sync == SYNC_AGENT) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  return last;
}

// Copy X[0:rows_p][k0:k0+win) into the LDS window (row stride d.xrow), zero
// outside [0,M) x [k0,kend).
__device__ __forceinline__ void stage_x(const StageDesc& d, uint16_t* xs, int rows_p, int k0,
                                        int kend, Rsrc xr) {
  const int cpr = d.win >> 3;
  const int total = rows_p * cpr;
#pragma unroll 4
  for (int q = threadIdx.x; q < total; q += blockDim.x) {
    const int row = q / cpr;
    const int cc = q - row * cpr;
    const int k = k0 + cc * 8;
    const bool valid = row < d.M && k < kend;
    const unsigned off = valid ? ((unsigned)row * (unsigned)d.ldx + (unsigned)k) * 2u : d.x_bytes;
    *(u4*)(xs + row * d.xrow + cc * 8) = ld16<0>(xr, off);
  }
}

// Store one output element according to the stage's mode.  Out-of-range
// elements are dropped by the buffer range check (off = extent).
__device__ __forceinline__ void store_out(const StageDesc& d, Rsrc yr, Rsrc y2r, bool ok, int m,
                                          int col, float v) {
  const unsigned e = (unsigned)m * (unsigned)d.ldy + (unsigned)col;
  if (d.mode == OUT_F32) {
    st_f32<kAuxNt>(yr, ok ? e * 4u : d.y_bytes, v);
  } else {
    st_u16<kAuxNt>(yr, ok ? e * 2u : d.y_bytes, bf16_bits(v));
    if (d.mode == OUT_BF16_F32) st_f32<kAuxNt>(y2r, ok ? e * 4u : d.y2_bytes, v);
  }
}

// ------------------------------------------------------------------ dot2
struct NoHook {
  __device__ bool operator()() const { return true; }
};

// pre_x() runs after the first weight loads are in flight and before X is
// staged; the chain waits there for the stage that produces X.  Returning
// false abandons the stage.
template <int M, int G, int P, typename Hook = NoHook>
__device__ void dot2_stage(const StageDesc& d, uint16_t* xs, int xcd, int slot, int nslots,
                           Hook pre_x = Hook()) {
  constexpr int V = pow2_at_least(G * M);
  static_assert(V <= 64, "G*M must fit one wave");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_my = d.items > slot ? (d.items - slot + nslots - 1) / nslots : 0;
  if (n_my <= 0) return;
  const int total = n_my * d.steps;
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const Rsrc pr = make_rsrc(d.part, d.part_bytes);
  const unsigned aux = d.w_aux;

  u4 ring[P][G];
  float acc[G][M];
#pragma unroll
  for (int c = 0; c < G; ++c)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[c][m] = 0.f;

  int i_ord = 0, i_t = 0;  // issue cursor
  auto issue = [&](u4(&dst)[G]) {
    if (i_ord < n_my) {
      const int item = slot + i_ord * nslots;
      const int s = item / d.NB;
      const int b = item - s * d.NB;
      const int k0 = s * d.KS;
      const int kend = min(d.K, k0 + d.KS);
      const int k = k0 + i_t * kDot2KStep + lane * 8;
      const int colb = xc0 + b * d.CB + wave * G;
#pragma unroll
      for (int c = 0; c < G; ++c) {
        const int col = colb + c;
        const bool valid = col < xc1 && k < kend;
        const unsigned off = valid ? ((unsigned)col * (unsigned)d.K + (unsigned)k) * 2u : d.w_bytes;
        dst[c] = ld16_pol(wr, off, aux);
      }
    }
    if (++i_t == d.steps) { i_t = 0; ++i_ord; }
  };

  auto x_window = [&](int ord) {
    const int item = slot + ord * nslots;
    const int s = item / d.NB;
    stage_x(d, xs, M, s * d.KS, min(d.K, s * d.KS + d.KS), xr);
  };

  auto epilogue = [&](int ord) {
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = 0.f;
#pragma unroll
    for (int c = 0; c < G; ++c)
#pragma unroll
      for (int m = 0; m < M; ++m) v[c * M + m] = acc[c][m];
    float r = wave_reduce_scatter<V>(v, lane);
    constexpr int grp = 64 / V;
    const int idx = lane / grp;
    const bool owner = (lane % grp) == 0 && idx < G * M;
    const int c = idx / M, m = idx - (idx / M) * M;
    const int item = slot + ord * nslots;
    const int s = item / d.NB;
    const int b = item - s * d.NB;
    const int col = xc0 + b * d.CB + wave * G + c;
    if (d.S > 1) {
      const int tile = (xcd * d.NB + b) * (d.CB / G) + wave;
      const unsigned base = (unsigned)tile * (unsigned)d.S;
      st_f32<0>(pr, owner ? ((base + s) * (unsigned)(G * M) + idx) * 4u : d.part_bytes, r);
      if (!wave_arrive(d.ctr + tile, d.S, d.sync, lane)) return;
      float t = 0.f;
      for (int q = 0; q < d.S; ++q) {
        float pv;
        if (q == s) {
          pv = r;
        } else {
          const unsigned off = owner ? ((base + q) * (unsigned)(G * M) + idx) * 4u : d.part_bytes;
          pv = d.sync == SYNC_XCD
                   ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)off, 0, kAuxSc1))
                   : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)off, 0, 0));
        }
        t += pv;
      }
      r = t;
    }
    store_out(d, yr, y2r, owner && col < xc1 && m < d.M, m, col, r);
  };

#pragma unroll
  for (int p = 0; p < P; ++p) issue(ring[p]);
  if (!pre_x()) return;
  x_window(0);
  __syncthreads();

  int c_ord = 0, c_t = 0;
  int cur_s = slot / d.NB;
  for (int T = 0; T < total; T += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (T + p < total) {
        u4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = *(const u4*)(xs + m * d.xrow + c_t * kDot2KStep + lane * 8);
#pragma unroll
        for (int c = 0; c < G; ++c)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[c][m] = dot8(ring[p][c], xv[m], acc[c][m]);
        issue(ring[p]);
        if (++c_t == d.steps) {
          epilogue(c_ord);
#pragma unroll
          for (int c = 0; c < G; ++c)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[c][m] = 0.f;
          c_t = 0;
          ++c_ord;
          if (c_ord < n_my) {
            const int s_new = (slot + c_ord * nslots) / d.NB;
            if (s_new != cur_s) {
              __syncthreads();
              x_window(c_ord);
              __syncthreads();
              cur_s = s_new;
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ MFMA
// NT n-tiles of 16 columns per wave (PAIRED: tile 0 = gate rows, tile 1 = the
// matching up rows pair_off further), MT m-tiles of 16 rows.
// Lane l: column l%16 of an n-tile, row l%16 of an m-tile, K group l/16.
// Within a 64-wide k-step, lane group g reads k = 16g + 8h + (0..7) for
// halves h = 0, 1, so each weight row's 128 bytes are one full cache line
// spread over the two loads; A (from LDS) uses the same k slots, which is all
// the dot product needs.
template <int MT, int NT, int P, bool PAIRED, typename Hook = NoHook>
__device__ void mfma_stage(const StageDesc& d, uint16_t* xs, int xcd, int slot, int nslots,
                           Hook pre_x = Hook()) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int n_my = d.items > slot ? (d.items - slot + nslots - 1) / nslots : 0;
  if (n_my <= 0) return;
  const int total = n_my * d.steps;
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const Rsrc pr = make_rsrc(d.part, d.part_bytes);
  const unsigned aux = d.w_aux;
  constexpr int TW = PAIRED ? 16 : 16 * NT;  // distinct output columns per wave

  u4 ring[P][NT][2];
  f4 acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = f4{0.f, 0.f, 0.f, 0.f};

  int i_ord = 0, i_t = 0;
  auto issue = [&](u4(&dst)[NT][2]) {
    if (i_ord < n_my) {
      const int item = slot + i_ord * nslots;
      const int s = item / d.NB;
      const int b = item - s * d.NB;
      const int k0 = s * d.KS;
      const int kend = min(d.K, k0 + d.KS);
      const int colb = xc0 + b * d.CB + wave * TW;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int col = PAIRED ? colb + r16 : colb + 16 * j + r16;
        const unsigned row = PAIRED ? (unsigned)(col + j * d.pair_off) : (unsigned)col;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = k0 + i_t * kMfmaKStep + 16 * g4 + 8 * h;
          const bool valid = col < xc1 && k < kend;
          const unsigned off = valid ? (row * (unsigned)d.K + (unsigned)k) * 2u : d.w_bytes;
          dst[j][h] = ld16_pol(wr, off, aux);
        }
      }
    }
    if (++i_t == d.steps) { i_t = 0; ++i_ord; }
  };

  auto x_window = [&](int ord) {
    const int item = slot + ord * nslots;
    const int s = item / d.NB;
    stage_x(d, xs, 16 * MT, s * d.KS, min(d.K, s * d.KS + d.KS), xr);
  };

  auto emit = [&](int colb, int j, int i, f4 v, f4 vu) {
    const int col = colb + (PAIRED ? 0 : 16 * j) + r16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * i + 4 * g4 + e;
      const bool ok = m < d.M && col < xc1;
      if (PAIRED) {
        store_out(d, yr, y2r, ok, m, col, silu_mul(v[e], vu[e]));
      } else {
        store_out(d, yr, y2r, ok, m, col, v[e]);
      }
    }
  };

  auto epilogue = [&](int ord) {
    const int item = slot + ord * nslots;
    const int s = item / d.NB;
    const int b = item - s * d.NB;
    const int colb = xc0 + b * d.CB + wave * TW;
    if (d.S > 1) {
      constexpr unsigned TILE = NT * MT * 256;  // floats per wave tile
      const int tile = (xcd * d.NB + b) * (d.CB / TW) + wave;
      const unsigned base = (unsigned)tile * (unsigned)d.S;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          st_f4<0>(pr, (((base + s) * TILE) + (j * MT + i) * 256 + lane * 4) * 4u, acc[j][i]);
      if (!wave_arrive(d.ctr + tile, d.S, d.sync, lane)) return;
      f4 tot[NT][MT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) tot[j][i] = f4{0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < d.S; ++q) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            f4 pv;
            if (q == s) {
              pv = acc[j][i];
            } else {
              const unsigned off = (((base + q) * TILE) + (j * MT + i) * 256 + lane * 4) * 4u;
              pv = d.sync == SYNC_XCD ? ld_f4<kAuxSc1>(pr, off) : ld_f4<0>(pr, off);
            }
            tot[j][i] += pv;
          }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (PAIRED) {
          emit(colb, 0, i, tot[0][i], tot[1][i]);
        } else {
#pragma unroll
          for (int j = 0; j < NT; ++j) emit(colb, j, i, tot[j][i], tot[j][i]);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (PAIRED) {
        emit(colb, 0, i, acc[0][i], acc[1][i]);
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) emit(colb, j, i, acc[j][i], acc[j][i]);
      }
    }
  };

#pragma unroll
  for (int p = 0; p < P; ++p) issue(ring[p]);
  if (!pre_x()) return;
  x_window(0);
  __syncthreads();

  int c_ord = 0, c_t = 0;
  int cur_s = slot / d.NB;
  for (int T = 0; T < total; T += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (T + p < total) {
        const uint16_t* xb = xs + r16 * d.xrow + c_t * kMfmaKStep + 16 * g4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 xa[MT];
#pragma unroll
          for (int i = 0; i < MT; ++i)
            xa[i] = __builtin_bit_cast(bf16x8, *(const u4*)(xb + 16 * i * d.xrow + 8 * h));
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const bf16x8 wb = __builtin_bit_cast(bf16x8, ring[p][j][h]);
#pragma unroll
            for (int i = 0; i < MT; ++i)
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], wb, acc[j][i], 0, 0, 0);
          }
        }
        issue(ring[p]);
        if (++c_t == d.steps) {
          epilogue(c_ord);
#pragma unroll
          for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[j][i] = f4{0.f, 0.f, 0.f, 0.f};
          c_t = 0;
          ++c_ord;
          if (c_ord < n_my) {
            const int s_new = (slot + c_ord * nslots) / d.NB;
            if (s_new != cur_s) {
              __syncthreads();
              x_window(c_ord);
              __syncthreads();
              cur_s = s_new;
            }
          }
        }
      }
    }
  }
}

}  // namespace sg
