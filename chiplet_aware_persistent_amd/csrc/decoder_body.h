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
#include "chain_body.h"

namespace sg {

constexpr int kAttnPos = 64;  // positions per attention unit (one per lane)

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
// the QKV output).  Lane i scores position 64c + i against the GRP query heads
// of g (v_dot2 over the head dimension against the queries staged in LDS),
// the wave takes the softmax of its 64 scores per head and accumulates
// sum_t p_t v_t with each lane holding two of the HD value dimensions.  The
// unit writes its (max, sum, accumulator) per head; the last of a (m, g)'s
// units to arrive (arrival counter, old value nchunk - 1) combines them in
// chunk order, so the result does not depend on timing, and writes bf16
// o[m][(g GRP + j) HD + i].
template <int GRP, int HD, typename Hook>
__device__ __forceinline__ bool gqa_stage(const ChainArgs& a, int l, uint16_t* lds, int xcd, int slot, int nslots,
                                          Hook pre) {
  static_assert(HD == 128, "two head dimensions per lane");
  if (!pre()) return false;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwv = (int)(blockDim.x >> 6);
  const int M = a.M, Hkv = a.Hkv, T = a.T, nch = a.nchunk;
  const int qcols = a.Hq * HD, ld = qcols + 2 * Hkv * HD;
  const uint16_t* qkv = a.act + (size_t)l * a.act_layer_elems + a.off_qkv;
  uint16_t* out = a.act + (size_t)l * a.act_layer_elems + a.off_o;
  const size_t cache_layer = (size_t)M * Hkv * T * HD;
  const Rsrc kr = make_rsrc(a.kc + (size_t)l * cache_layer, (unsigned)(cache_layer * 2));
  const Rsrc vr = make_rsrc(a.vc + (size_t)l * cache_layer, (unsigned)(cache_layer * 2));
  const unsigned qkv_bytes = (unsigned)((size_t)M * ld * 2);
  const Rsrc qr = make_rsrc(qkv, qkv_bytes);
  const Rsrc orr = make_rsrc(out, (unsigned)((size_t)M * qcols * 2));
  constexpr int PL = GRP * (HD + 2);  // floats of one unit's partial
  const Rsrc pr = make_rsrc(a.apart, (unsigned)((size_t)M * Hkv * nch * PL * 4));
  const float scale = 1.0f / __builtin_sqrtf((float)HD);
  // Per wave: the GRP query rows (GRP x HD bf16) and the 64 x GRP weights.
  uint16_t* qs = lds + wave * (GRP * HD + 2 * kAttnPos * GRP);
  float* ps = (float*)(qs + GRP * HD);
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
    // Queries of heads g GRP .. g GRP + GRP - 1 into LDS (contiguous in the row).
    static_assert(GRP * HD * 2 % 1024 == 0, "whole kilobytes of queries");
#pragma unroll
    for (int b = 0; b < GRP * HD * 2 / 1024; ++b) {
      const unsigned off = ((unsigned)m * ld + (unsigned)g * GRP * HD) * 2u + (unsigned)(b * 1024 + lane * 16);
      *(u4*)((char*)qs + b * 1024 + lane * 16) = ld16<0>(qr, off);
    }
    // This lane's key row: position t = 64c + lane (cache for t < T, the
    // new key for t == T, zeros past T).
    const int t = c * kAttnPos + lane;
    const unsigned crow = ((((unsigned)m * Hkv + g) * (unsigned)T + (unsigned)t) * HD) * 2u;
    const unsigned nrow = ((unsigned)m * ld + (unsigned)qcols + (unsigned)g * HD) * 2u;
    u4 kv[HD / 8];
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) {
      const u4 a0 = ld16<0>(kr, t < T ? crow + i * 16u : (unsigned)(cache_layer * 2));
      const u4 a1 = ld16<0>(qr, t == T ? nrow + i * 16u : qkv_bytes);
      kv[i] = a0 | a1;
    }
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
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      float v = live ? s[j] * scale : -__builtin_huge_valf();
      float mm = v;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
      const float p = live ? __builtin_amdgcn_exp2f((v - mm) * 1.4426950408889634f) : 0.f;
      float sm = p;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
      mx[j] = mm;
      lsum[j] = sm;
      ps[lane * GRP + j] = p;
    }
    // sum_t p_t v_t: lane holds value dimensions 2 lane, 2 lane + 1.
    float acc[GRP][2];
#pragma unroll
    for (int j = 0; j < GRP; ++j) acc[j][0] = acc[j][1] = 0.f;
    const unsigned vcol = (unsigned)lane * 4u;
    const int tn = min(kAttnPos, T + 1 - c * kAttnPos);  // live positions of the unit
    for (int t0 = 0; t0 < tn; t0 += 16) {
      unsigned vv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tt = c * kAttnPos + t0 + i;
        const unsigned co = ((((unsigned)m * Hkv + g) * (unsigned)T + (unsigned)tt) * HD) * 2u + vcol;
        const unsigned no = ((unsigned)m * ld + (unsigned)qcols + (unsigned)(Hkv + g) * HD) * 2u + vcol;
        const unsigned a0 = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)(tt < T ? co : (unsigned)(cache_layer * 2)), 0, 0);
        const unsigned a1 = __builtin_amdgcn_raw_buffer_load_b32(qr, (int)(tt == T ? no : qkv_bytes), 0, 0);
        vv[i] = a0 | a1;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bf16x2 vb = __builtin_bit_cast(bf16x2, vv[i]);
        const float v0 = (float)vb[0], v1 = (float)vb[1];
#pragma unroll
        for (int j = 0; j < GRP; ++j) {
          const float p = ps[(t0 + i) * GRP + j];  // zero past the live positions
          acc[j][0] += p * v0;
          acc[j][1] += p * v1;
        }
      }
    }
    // The unit's partial: per head HD accumulator values, then max and sum.
    const unsigned pbase = (unsigned)((((size_t)m * Hkv + g) * nch + c) * PL);
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const unsigned e = pbase + j * (HD + 2);
      st_f32<0>(pr, (e + 2 * lane) * 4u, acc[j][0]);
      st_f32<0>(pr, (e + 2 * lane + 1) * 4u, acc[j][1]);
      if (lane == 0) {
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
    // Lane cc holds chunk cc's max and sum (nch <= 64); the accumulators are
    // read 16 chunks at a time.  Every sum runs in a fixed order.
    const unsigned base = (unsigned)(((size_t)m * Hkv + g) * nch * PL);
    const unsigned pext = (unsigned)((size_t)M * Hkv * nch * PL * 4);
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const unsigned ej = base + lane * PL + j * (HD + 2);
      const float mc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     pr, (int)(lane < nch ? (ej + HD) * 4u : pext), 0, kAuxSc1));
      const float lc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     pr, (int)(lane < nch ? (ej + HD + 1) * 4u : pext), 0, kAuxSc1));
      float gm = lane < nch ? mc : -__builtin_huge_valf();
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
      const float f = lane < nch ? __builtin_amdgcn_exp2f((mc - gm) * 1.4426950408889634f) : 0.f;
      float L = lc * f;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
      float o0 = 0.f, o1 = 0.f;
      for (int c0 = 0; c0 < nch; c0 += 16) {
        float a0[16], a1[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const unsigned e = base + (unsigned)(c0 + i) * PL + j * (HD + 2) + 2 * lane;
          const bool in = c0 + i < nch;
          a0[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)(in ? e * 4u : pext), 0, kAuxSc1));
          a1[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (int)(in ? (e + 1) * 4u : pext), 0, kAuxSc1));
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float fi = __shfl(f, c0 + i);  // zero past nch
          o0 += a0[i] * fi;
          o1 += a1[i] * fi;
        }
      }
      const unsigned oc = ((unsigned)m * qcols + (unsigned)(g * GRP + j) * HD + 2u * lane) * 2u;
      const unsigned pk = (unsigned)bf16_bits(o0 / L) | ((unsigned)bf16_bits(o1 / L) << 16);
      __builtin_amdgcn_raw_buffer_store_b32(pk, orr, (int)oc, 0, kAuxNt);
    }
  }
  return true;
}

// PATH 1: MFMA stages (A = MT, B = NT); PATH 0: dot2 stages (A = M, B = G).
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
