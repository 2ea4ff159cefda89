// The whole decoder layer in one persistent launch: the projection chain's
// machinery (per-XCD column partition, stage streams, two-level completion
// counters, weights prefetched across each stage wait) with the operators
// between the projections added as stages or fused into them.
//
// Per layer l, on the residual stream x (Fleet reading note, TL;DR and
// Summary: about seven operators per layer; section 1: a Qwen3-8B-shaped
// decoder with grouped-query attention):
//   event 5l+0  qkv = bf16(rmsnorm(x) w_attn . Wqkv^T)   the norm is applied to
//               each workgroup's staged X window in LDS (RmsNormX)
//   event 5l+1  o   = bf16(attention(q, K|k, V|v))       gqa_stage
//   event 5l+2  x1  = bf16(x + o . Wo^T)                 residual in the epilogue
//   event 5l+3  a   = bf16(silu(g) u), [g|u] = rmsnorm(x1) w_mlp . Wgu^T
//   event 5l+4  x'  = bf16(x1 + a . Wdown^T)             (+ fp32 for the last layer)
#pragma once
#include <type_traits>

#include "chain_body.h"

namespace sg {

constexpr int kAttnPos = 64;  // positions per attention unit (one per lane)
constexpr int kAttnWaveLds = 4 * 128 * 2 + kAttnPos * 4 * 4 + kAttnPos * 128 * 2;  // bytes of LDS per wave

// Two dwords.  A plain struct: an ext_vector_type(2) built from two adjacent
// dword buffer loads compiled here to one dword load copied into both halves
// (buffer_load_dword, then v_mov of the same register), and so did the
// 8-byte buffer-load builtin; the struct's two loads become one
// buffer_load_dwordx2.
struct U2 {
  unsigned x, y;
};

// 8 bytes (off at or past the extent: zeros).
template <int AUX>
__device__ __forceinline__ U2 ld8(Rsrc r, unsigned off) {
  return U2{__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX),
            __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4u), 0, AUX)};
}

// Four bf16 (two dwords, element 0 in the low half of x) to fp32: a bf16 is
// the upper half of the fp32 with the same value, so shifts and masks
// convert exactly.
__device__ __forceinline__ f4 bf16x4_to_f4(U2 w) {
  return f4{__builtin_bit_cast(float, w.x << 16), __builtin_bit_cast(float, w.x & 0xffff0000u),
            __builtin_bit_cast(float, w.y << 16), __builtin_bit_cast(float, w.y & 0xffff0000u)};
}

// RMSNorm of the rows of X applied to a staged X window (rows [0, rows) x K
// values [k0, k0 + win), row stride xrow): every workgroup computes the
// reciprocal RMS of each row from the full row in global memory (fp32 sum of
// squares, one wave per row), then scales its window in place:
// x = bf16(x * rstd[row] * w[k]).  Called after the window's loads are issued;
// it waits for them itself.
struct RmsNormX {
  static constexpr bool active = true;
  const uint16_t* x;  // [M][K] bf16, the stage input
  const uint16_t* w;  // [K] bf16, the norm weight
  float* rstd;        // LDS, M floats
  int M, K;
  float eps;
  __device__ void operator()(uint16_t* xs, int rows, int xrow, int k0, int win) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = (int)(blockDim.x >> 6);
    const Rsrc xr = make_rsrc(x, (unsigned)M * (unsigned)K * 2u);
    for (int r = wave; r < M; r += nw) {
      float ss = 0.f;
      for (int k = lane * 8; k < K; k += 512) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, ld16<0>(xr, ((unsigned)r * (unsigned)K + (unsigned)k) * 2u));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float f = (float)v[i];
          ss += f * f;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      if (lane == 0) rstd[r] = 1.0f / __builtin_sqrtf(ss / (float)K + eps);
    }
    wait_vm0();  // the window's loads and the rows read above
    __syncthreads();
    const Rsrc wr = make_rsrc(w, (unsigned)K * 2u);
    const int groups = win >> 3;  // 8 values per group; win, xrow and k0 are multiples of 8
    for (int i = threadIdx.x; i < rows * groups; i += blockDim.x) {
      const int r = i / groups;
      const int c = (i - r * groups) * 8;
      const int k = k0 + c;
      if (k >= K) continue;  // zero padding past K stays zero
      uint16_t* p = xs + r * xrow + c;
      const bf16x8 xv = *(const bf16x8*)p;
      const bf16x8 wv = __builtin_bit_cast(bf16x8, ld16<0>(wr, (unsigned)k * 2u));
      const float s = rstd[r];
      bf16x8 o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = (__bf16)((float)xv[j] * s * (float)wv[j]);
      *(bf16x8*)p = o;
    }
    __syncthreads();
  }
};

// Grouped-query decode attention of layer l (event 5l+1).  Key/value head g
// belongs to XCD g mod 8, so all the work on one head, and its combine,
// stays in that XCD's L2.  A unit is one wave: sequence m, head g, positions
// [64c, 64c + 64) of the T cached ones and the new one (position T, read from
// the QKV output).  The unit issues all its loads at once, so it costs about
// one memory round trip: lane i's key row 64c + i into registers, and the
// 64 value rows into the wave's LDS with buffer-to-LDS loads (16 KB, no
// registers).  Lane i scores its position against the GRP query heads of g
// (v_dot2 over the head dimension against the queries staged in LDS), the
// wave takes the softmax of its 64 scores per head, then sums p_t v_t from
// LDS in two halves (lanes 0-31 positions 64c + r, lanes 32-63 positions
// 64c + 32 + r, each lane four value dimensions) and adds the halves.  The
// unit writes its (max, sum, accumulator) per head; the last of a (m, g)'s
// units to arrive (arrival counter, old value nchunk - 1) combines them in
// chunk order, so the result does not depend on timing, and writes bf16
// o[m][(g GRP + j) HD + i].  The combine loads every chunk's max and sum of
// all heads at once and keeps the next batch of accumulators in flight while
// it adds the current one.
template <int GRP, int HD, typename Hook>
__device__ __forceinline__ bool gqa_stage(const ChainArgs& a, int l, uint16_t* lds, int xcd, int slot, int nslots,
                                          Hook pre) {
  static_assert(HD == 128, "four head dimensions per lane and half");
  static_assert(GRP == 4 && GRP * HD * 2 == 1024, "one kilobyte of queries per unit");
  if (!pre()) return false;
  const int wave = threadIdx.x >> 6;
  const int nwv = (int)(blockDim.x >> 6);
  const int M = a.M, Hkv = a.Hkv, T = a.T, nch = a.nchunk;
  const int qcols = a.Hq * HD, ld = qcols + 2 * Hkv * HD;
  const uint16_t* qkv = a.act + (size_t)l * a.act_layer_elems + a.off_qkv;
  uint16_t* out = a.act + (size_t)l * a.act_layer_elems + a.off_o;
  const size_t cache_layer = (size_t)M * Hkv * T * HD;
  const unsigned cext = (unsigned)(cache_layer * 2);
  const Rsrc kr = make_rsrc(a.kc + (size_t)l * cache_layer, cext);
  const Rsrc vr = make_rsrc(a.vc + (size_t)l * cache_layer, cext);
  const unsigned qkv_bytes = (unsigned)((size_t)M * ld * 2);
  const Rsrc qr = make_rsrc(qkv, qkv_bytes);
  const Rsrc orr = make_rsrc(out, (unsigned)((size_t)M * qcols * 2));
  constexpr int PL = GRP * (HD + 2);  // floats of one unit's partial
  const unsigned pext = (unsigned)((size_t)M * Hkv * nch * PL * 4);
  const Rsrc pr = make_rsrc(a.apart, pext);
  const float scale = 1.0f / __builtin_sqrtf((float)HD);
  constexpr float kLog2e = 1.4426950408889634f;
  // Per wave (kAttnWaveLds bytes): the GRP query rows (GRP x HD bf16), the
  // 64 x GRP weights and the 64 value rows (64 x HD bf16).
  static_assert(kAttnWaveLds == GRP * HD * 2 + kAttnPos * GRP * 4 + kAttnPos * HD * 2, "attention LDS layout");
  uint16_t* qs = (uint16_t*)((char*)lds + wave * kAttnWaveLds);
  float* ps = (float*)(qs + GRP * HD);
  uint16_t* vs = (uint16_t*)(ps + kAttnPos * GRP);
  const int hpx = (Hkv + kXcds - 1) / kXcds;  // key/value heads per XCD
  const int units = hpx * M * nch;
  const int nwx = nslots * nwv;
  for (int u = slot * nwv + wave; u < units; u += nwx) {
    const int gi = u / (M * nch);
    const int rem = u - gi * (M * nch);
    const int m = rem / nch;
    const int c = rem - m * nch;
    const int g = xcd + kXcds * gi;
    if (g >= Hkv) continue;  // uniform over the wave
    // The lane index, opaque to the compiler inside the unit: otherwise it
    // hoists the dozens of per-lane load offsets out of the layer loop and
    // keeps them in registers through every stage of the launch.
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int hf = lane >> 5;        // value half: positions [32 hf, 32 hf + 32) of the unit
    const int dq = 4 * (lane & 31);  // the lane's first value dimension
    const int t = c * kAttnPos + lane;
    const unsigned hrow = ((unsigned)m * Hkv + g) * (unsigned)T;  // first cache row of (m, g)
    const bool has_new = T >= c * kAttnPos && T < (c + 1) * kAttnPos;  // uniform: the chunk holding position T
    // All loads of the unit, oldest first: queries, key rows (the cache for
    // t < T, zeros past it; the new key for t == T only in the last chunk),
    // value dimensions [dq, dq + 4) of the 32 positions of the lane's half
    // (and of the new position).
    const u4 qv = ld16<0>(qr, ((unsigned)m * ld + (unsigned)g * GRP * HD) * 2u + (unsigned)lane * 16u);
    u4 kv[HD / 8];
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) kv[i] = ld16<0>(kr, t < T ? (hrow + (unsigned)t) * HD * 2u + i * 16u : cext);
    // Value rows to LDS: kilobyte i holds positions 64c + 4i .. 64c + 4i + 3
    // (lane l: position 4i + l/16, dimensions 8 (l % 16) .. + 7).
#pragma unroll
    for (int i = 0; i < kAttnPos * HD * 2 / 1024; ++i) {
      const int tt = c * kAttnPos + 4 * i + (lane >> 4);
      const unsigned off = tt < T ? ((hrow + (unsigned)tt) * HD + 8u * (unsigned)(lane & 15)) * 2u : cext;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)((char*)vs + i * 1024),
                                               16, off, 0, 0, 0);
    }
    U2 vnew = {0u, 0u};
    if (has_new) {
      const unsigned nkrow = ((unsigned)m * ld + (unsigned)qcols + (unsigned)g * HD) * 2u;
      const unsigned nvrow = ((unsigned)m * ld + (unsigned)qcols + (unsigned)(Hkv + g) * HD) * 2u;
#pragma unroll
      for (int i = 0; i < HD / 8; ++i) kv[i] |= ld16<0>(qr, t == T ? nkrow + i * 16u : qkv_bytes);
      vnew = ld8<0>(qr, hf == 0 ? nvrow + (unsigned)dq * 2u : qkv_bytes);
    }
    *(u4*)((char*)qs + lane * 16) = qv;
    __builtin_amdgcn_wave_barrier();
    float s[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) s[j] = 0.f;
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, kv[i]);
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const bf16x8 qb = *(const bf16x8*)(qs + j * HD + i * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 kp = {kb[2 * e], kb[2 * e + 1]};
          const bf16x2 qp = {qb[2 * e], qb[2 * e + 1]};
          s[j] = __builtin_amdgcn_fdot2_f32_bf16(kp, qp, s[j], false);
        }
      }
    }
    const bool live = t <= T;
    float mx[GRP], lsum[GRP];
    f4 pl;
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const float v = live ? s[j] * scale : -__builtin_huge_valf();
      float mm = v;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
      const float p = live ? __builtin_amdgcn_exp2f((v - mm) * kLog2e) : 0.f;
      float sm = p;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
      mx[j] = mm;
      lsum[j] = sm;
      pl[j] = p;
    }
    *(f4*)(ps + lane * GRP) = pl;
    __builtin_amdgcn_wave_barrier();
    // sum_t p_t v_t over the lane's half (zero weights past T), the new
    // position's row (half 0), then the two halves added.
    wait_vm0();  // the value rows are in LDS
    f4 acc[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const U2 vr2 = *(const U2*)(vs + (32 * hf + r) * HD + dq);
      const f4 v = bf16x4_to_f4(vr2);
      const f4 p4 = *(const f4*)(ps + (32 * hf + r) * GRP);
#pragma unroll
      for (int j = 0; j < GRP; ++j) acc[j] += p4[j] * v;
    }
    if (has_new) {
      const f4 v = bf16x4_to_f4(vnew);
      const f4 p4 = *(const f4*)(ps + (T - c * kAttnPos) * GRP);
#pragma unroll
      for (int j = 0; j < GRP; ++j) acc[j] += p4[j] * v;  // zero in half 1
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] += __shfl_xor(acc[j][e], 32);
    // The unit's partial: per head HD accumulator values, then max and sum.
    const unsigned pbase = (unsigned)((((size_t)m * Hkv + g) * nch + c) * PL);
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const unsigned e = pbase + j * (HD + 2);
      if (hf == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) st_f32<0>(pr, (e + dq + q) * 4u, acc[j][q]);
      }
      if (lane == 32) {
        st_f32<0>(pr, (e + HD) * 4u, mx[j]);
        st_f32<0>(pr, (e + HD + 1) * 4u, lsum[j]);
      }
    }
    // Arrival: the XCD-local split-K protocol (all units of (m, g) run on
    // this XCD).  The owner adds the chunks in order.
    splitk_release(SYNC_XCD);
    unsigned* ctr = a.actr + m * Hkv + g;
    const unsigned old = splitk_bump(ctr, lane);
    if (!splitk_own(ctr, old, nch, SYNC_XCD, lane)) continue;
    // Lane cc holds chunk cc's max and sum of every head (nch <= 64).
    const unsigned base = (unsigned)(((size_t)m * Hkv + g) * nch * PL);
    float mc[GRP], lc[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const unsigned ej = base + lane * PL + j * (HD + 2);
      mc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            pr, (int)(lane < nch ? (ej + HD) * 4u : pext), 0, kAuxSc1));
      lc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            pr, (int)(lane < nch ? (ej + HD + 1) * 4u : pext), 0, kAuxSc1));
    }
    // Accumulators of head j, chunks [16 h, 16 h + 16): the lane's two values
    // (dimensions 2 lane, 2 lane + 1) per chunk.  Batches in (head, chunk
    // group) order alternate between two register sets; each is issued before
    // the one ahead of it is added, and in-order returns leave it in flight.
    auto issue = [&](U2(&dst)[16], int j, int h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cc = 16 * h + i;
        const unsigned e = base + (unsigned)cc * PL + j * (HD + 2) + 2 * lane;
        dst[i] = ld8<kAuxSc1>(pr, cc < nch ? e * 4u : pext);
      }
    };
    float o0[GRP], o1[GRP], L[GRP];
    auto combine = [&](auto nbc) {
      constexpr int NB = decltype(nbc)::value;  // chunk groups of 16 per head (nch <= 16 NB)
      U2 buf[2][16];
      issue(buf[0], 0, 0);
      float f[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        float gm = lane < nch ? mc[j] : -__builtin_huge_valf();
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
        f[j] = lane < nch ? __builtin_amdgcn_exp2f((mc[j] - gm) * kLog2e) : 0.f;
        float sl = lc[j] * f[j];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sl += __shfl_xor(sl, o);
        L[j] = sl;
        o0[j] = o1[j] = 0.f;
      }
#pragma unroll
      for (int b = 0; b < NB * GRP; ++b) {
        const int j = b / NB, h = b % NB;
        if (b + 1 < NB * GRP) issue(buf[(b + 1) & 1], (b + 1) / NB, (b + 1) % NB);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float fi = __shfl(f[j], 16 * h + i);  // zero past nch
          o0[j] += __builtin_bit_cast(float, buf[b & 1][i].x) * fi;
          o1[j] += __builtin_bit_cast(float, buf[b & 1][i].y) * fi;
        }
      }
    };
    const int ng = (nch + 15) / 16;
    if (ng == 1) {
      combine(std::integral_constant<int, 1>{});
    } else if (ng == 2) {
      combine(std::integral_constant<int, 2>{});
    } else if (ng == 3) {
      combine(std::integral_constant<int, 3>{});
    } else {
      combine(std::integral_constant<int, 4>{});
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const unsigned oc = ((unsigned)m * qcols + (unsigned)(g * GRP + j) * HD + 2u * lane) * 2u;
      const unsigned pk = (unsigned)bf16_bits(o0[j] / L[j]) | ((unsigned)bf16_bits(o1[j] / L[j]) << 16);
      __builtin_amdgcn_raw_buffer_store_b32(pk, orr, (int)oc, 0, kAuxNt);
    }
  }
  return true;
}

template <int PATH, int A, int B>
__global__ __launch_bounds__(512) void k_decoder(ChainArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ int sh_alive;
  __shared__ int sh_last;
  const int xcd = xcd_of_wg(a.status);
  const int slot = blockIdx.x >> 3;
  const int nslots = gridDim.x >> 3;
  if (threadIdx.x == 0) {
    const unsigned bit = slot < 32 ? 1u << slot : 0u;
    const unsigned old = __hip_atomic_fetch_or(a.claim + xcd, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bit == 0u || (old & bit))
      __hip_atomic_fetch_or(a.status, kStatusTopology, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  constexpr int kSpl = 5;
  float* rstd = (float*)((char*)lds + a.norm_off);
  bool alive = true;
  for (int l = 0; l < a.n_layers && alive; ++l) {
    uint16_t* act = a.act + (size_t)l * a.act_layer_elems;
    const uint16_t* xin = l == 0 ? a.x0 : a.act + (size_t)(l - 1) * a.act_layer_elems + a.off_x;
    const uint16_t* wn = a.wnorm + (size_t)l * 2 * a.d;
#pragma unroll
    for (int s = 0; s < kSpl; ++s) {
      if (!alive) break;
      const int e = kSpl * l + s;
      auto hook = [&]() -> bool {
        const bool ok = e == 0 ? true : wait_event(a, e - 1, xcd, slot, &sh_alive);
        stamp(a, e, 0);
        return ok;
      };
      if (s == 1) {
        alive = gqa_stage<4, 128>(a, l, lds, xcd, slot, nslots, hook);
      } else {
        StageDesc d = a.st[s == 0 ? 0 : s - 1];  // GEMM stage descriptor: QKV, O, gate_up, down
        RmsNormX nrm;
        nrm.rstd = rstd;
        nrm.M = a.M;
        nrm.K = a.d;
        nrm.eps = a.eps;
        if (s == 0) { d.X = xin; d.W = a.wq[l]; d.Y = act + a.off_qkv; nrm.x = xin; nrm.w = wn; }
        if (s == 2) { d.X = act + a.off_o; d.W = a.wo[l]; d.Y = act + a.off_x1; d.R = xin; }
        if (s == 3) { d.X = act + a.off_x1; d.W = a.wgu[l]; d.Y = act + a.off_a; nrm.x = act + a.off_x1; nrm.w = wn + a.d; }
        if (s == 4) {
          d.X = act + a.off_a; d.W = a.wdown[l]; d.Y = act + a.off_x; d.R = act + a.off_x1;
          if (l == a.n_layers - 1) { d.mode = OUT_BF16_F32; d.Y2 = a.y_f32; }
        }
        if constexpr (PATH == 1) {
          if (s == 3) {
            alive = mfma_stage<A, 2, true, kAuxNt, (A <= 2), decltype(hook), false, RmsNormX>(d, lds, xcd, slot, nslots,
                                                                                            hook, nrm);
          } else if (s == 0) {
            alive = mfma_stage<A, B, false, kAuxNt, (A <= 2), decltype(hook), false, RmsNormX>(d, lds, xcd, slot,
                                                                                             nslots, hook, nrm);
          } else {
            alive = mfma_stage<A, B, false, kAuxNt, (A <= 2)>(d, lds, xcd, slot, nslots, hook);
          }
        } else {
          if (s == 3) {
            alive = dot2_stage<A, B, kAuxNt, true, decltype(hook), RmsNormX>(d, lds, xcd, slot, nslots, hook, nrm);
          } else if (s == 0) {
            alive = dot2_stage<A, B, kAuxNt, false, decltype(hook), RmsNormX>(d, lds, xcd, slot, nslots, hook, nrm);
          } else {
            alive = dot2_stage<A, B, kAuxNt, false>(d, lds, xcd, slot, nslots, hook);
          }
        }
      }
      if (!alive) break;
      if (a.stamps) __syncthreads();
      stamp(a, e, 1);
      if (e + 1 < kSpl * a.n_layers) signal_event(a, e, xcd, nslots);
      __syncthreads();  // LDS reuse by the next stage
    }
  }
  // Finish as the chain does: the last workgroup resets the launch's counters.
  wait_vm0();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = old == gridDim.x - 1;
    if (sh_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (sh_last) {
    const int events = kSpl * a.n_layers;
    for (int i = threadIdx.x; i < a.gcopies * events; i += blockDim.x) a.gctr[i] = 0u;
    for (int i = threadIdx.x; i < kXcds * events; i += blockDim.x) {
      a.lctr[i] = 0u;
      a.xflag[i] = 0u;
    }
    if (threadIdx.x < kXcds) a.claim[threadIdx.x] = 0u;
    for (int s = 0; s < kChainStages; ++s) {
      const int n = a.st[s].nctr;
      for (int i = threadIdx.x; i < n; i += blockDim.x) a.st[s].ctr[i] = 0u;
    }
    for (int i = threadIdx.x; i < a.M * a.Hkv; i += blockDim.x) a.actr[i] = 0u;
    wait_vm0();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace sg
