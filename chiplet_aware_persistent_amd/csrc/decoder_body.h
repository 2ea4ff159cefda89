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
// Bytes of LDS per wave: queries, weights, value rows, and the new position's
// key and value rows.
constexpr int kAttnWaveLds = 4 * 128 * 2 + kAttnPos * 4 * 4 + kAttnPos * 128 * 2 + 2 * 128 * 2;

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
// belongs to XCD g mod 8, so all the work on one head stays in that XCD's L2.
// A (sequence m, head g) pair is split into S slices (S = 1 when an XCD has
// enough pairs to keep its workgroups busy, up to 8 for few); slice s is one
// workgroup and takes the chunks c = s, s + S, ... of 64 positions of the T
// cached ones and the new one (position T, read from the QKV output).  Its
// eight waves take those chunks in turn and each keeps a running softmax
// (max, sum and accumulator, rescaled as the max grows).  A chunk costs one
// memory round trip: the lane's key row 64c + lane into registers and the 64
// value rows into the wave's LDS with buffer-to-LDS loads, all issued at
// once; lane i scores its position against the GRP query heads of g (v_dot2
// over the head dimension against the queries in LDS), and p_t v_t is summed
// from LDS in two halves (lanes 0-31 positions 64c + r, lanes 32-63 positions
// 64c + 32 + r, four value dimensions per lane).  The waves' results meet in
// LDS and waves 0..GRP-1 add them in wave order, one head each.  With S > 1
// the slice's result goes to memory and the slice whose arrival completes
// the pair (XCD-local arrival counter, old value S - 1) adds the S results in
// slice order.  Every sum runs in a fixed order, so the output does not
// depend on timing.  Output: bf16 o[m][(g GRP + j) HD + i].
template <int GRP, int HD, typename Hook>
__device__ __forceinline__ bool gqa_stage(const ChainArgs& a, int l, uint16_t* lds, int xcd, int slot, int nslots,
                                          Hook pre) {
  static_assert(HD == 128, "four head dimensions per lane and half");
  static_assert(GRP == 4 && GRP * HD * 2 == 1024, "one kilobyte of queries per pair");
  constexpr int RL = HD + 2;  // floats of one head's result: accumulator, max, sum
  static_assert(GRP * RL * 4 <= kAttnPos * HD * 2, "a wave's result fits its value rows' LDS");
  const int wave = threadIdx.x >> 6;
  const int nwv = (int)(blockDim.x >> 6);
  const int M = a.M, Hkv = a.Hkv, T = a.T, nch = a.nchunk, S = a.attn_s;
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
  const unsigned pext = (unsigned)((size_t)M * Hkv * S * GRP * RL * 4);
  const Rsrc pr = make_rsrc(a.apart, pext);  // slice results [m][g][slice][head][RL]
  const float scale = 1.0f / __builtin_sqrtf((float)HD);
  constexpr float kLog2e = 1.4426950408889634f;
  auto wave_lds = [&](int w) { return (char*)lds + w * kAttnWaveLds; };
  uint16_t* qs = (uint16_t*)wave_lds(wave);
  float* ps = (float*)(qs + GRP * HD);
  uint16_t* vs = (uint16_t*)(ps + kAttnPos * GRP);
  const int vs_off = GRP * HD * 2 + kAttnPos * GRP * 4;  // byte offset of the value rows in a wave's LDS
  uint16_t* nk = vs + kAttnPos * HD;  // the new position's key row, then its value row
  uint16_t* nv = nk + HD;
  // With T a multiple of 64 the new position would be a chunk of its own and
  // cost its wave a third round trip.  Instead the wave that chunk falls to
  // loads the new key and value rows into LDS with its first loads and adds
  // the position after its cached chunks (the tail step below).
  const bool newsep = T % kAttnPos == 0;
  const int ncc = newsep ? nch - 1 : nch;  // chunks holding cached positions
  const int c_new = T / kAttnPos;
  const int hpx = (Hkv + kXcds - 1) / kXcds;
  const int tasks = hpx * M * S;  // (pair, slice), slice fastest
  // Value rows of a chunk to the wave's LDS: kilobyte i holds positions
  // 64c + 4i .. + 3 (lane l: position 4i + l/16, dimensions 8 (l % 16) .. + 7).
  auto issue_values = [&](int c, unsigned hrow, int ln) {
#pragma unroll
    for (int i = 0; i < kAttnPos * HD * 2 / 1024; ++i) {
      const int tt = c * kAttnPos + 4 * i + (ln >> 4);
      const unsigned off = tt < T ? ((hrow + (unsigned)tt) * HD + 8u * (unsigned)(ln & 15)) * 2u : cext;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)((char*)vs + i * 1024),
                                               16, off, 0, 0, 0);
    }
  };
  // The cache does not depend on the stage's input: the value rows of the
  // first chunk of the wave's first task go to LDS before the wait (the LDS
  // is free, every stage ends at a barrier), so their round trip overlaps
  // the previous stage.  They take no registers across the wait.
  bool vahead = false;
  if (slot < tasks) {
    const int pi = slot / S;
    const int sl = slot - pi * S;
    const int gi = pi / M;
    const int m = pi - gi * M;
    const int g = xcd + kXcds * gi;
    const int c = sl + S * wave;
    if (g < Hkv && c < ncc) {
      int ln = threadIdx.x & 63;
      asm volatile("" : "+v"(ln));
      issue_values(c, ((unsigned)m * Hkv + g) * (unsigned)T, ln);
      vahead = true;
    }
  }
  if (!pre()) return false;
  for (int task = slot; task < tasks; task += nslots) {
    const int pi = task / S;
    const int sl = task - pi * S;
    const int gi = pi / M;
    const int m = pi - gi * M;
    const int g = xcd + kXcds * gi;
    if (g >= Hkv) continue;  // uniform over the workgroup
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));  // keeps the per-lane offsets inside the loop
    const int hf = lane >> 5;
    const int dq = 4 * (lane & 31);
    const unsigned hrow = ((unsigned)m * Hkv + g) * (unsigned)T;
    const unsigned nkrow = ((unsigned)m * ld + (unsigned)qcols + (unsigned)g * HD) * 2u;
    const unsigned nvrow = ((unsigned)m * ld + (unsigned)qcols + (unsigned)(Hkv + g) * HD) * 2u;
    // The queries (one kilobyte) go to LDS by a buffer-to-LDS load, so their
    // round trip overlaps the first chunk's key loads.
    __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (__attribute__((address_space(3))) void*)qs, 16,
                                             ((unsigned)m * ld + (unsigned)g * GRP * HD) * 2u + (unsigned)lane * 16u,
                                             0, 0, 0);
    bool qpend = true;
    const bool tail = newsep && sl == c_new % S && wave == (c_new / S) % nwv;  // uniform
    if (tail) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (__attribute__((address_space(3))) void*)nk, 4,
                                               nkrow + (unsigned)lane * 4u, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (__attribute__((address_space(3))) void*)nv, 4,
                                               nvrow + (unsigned)lane * 4u, 0, 0, 0);
    }
    float mrun[GRP], lrun[GRP];
    f4 acc[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      mrun[j] = -__builtin_huge_valf();
      lrun[j] = 0.f;
      acc[j] = f4{0.f, 0.f, 0.f, 0.f};
    }
    for (int c = sl + S * wave; c < ncc; c += S * nwv) {
      asm volatile("" : "+v"(lane));  // and inside the chunk loop
      const int t = c * kAttnPos + lane;
      const bool has_new = T >= c * kAttnPos && T < (c + 1) * kAttnPos;  // uniform
      u4 kv[HD / 8];
#pragma unroll
      for (int i = 0; i < HD / 8; ++i) kv[i] = ld16<0>(kr, t < T ? (hrow + (unsigned)t) * HD * 2u + i * 16u : cext);
      if (!vahead) issue_values(c, hrow, lane);
      vahead = false;
      if (qpend) {
        // At least the 16 key loads were issued after the queries' load.
        wait_vm<HD / 8>();
        __builtin_amdgcn_wave_barrier();
        qpend = false;
      }
      U2 vnew = {0u, 0u};
      if (has_new) {
#pragma unroll
        for (int i = 0; i < HD / 8; ++i) kv[i] |= ld16<0>(qr, t == T ? nkrow + i * 16u : qkv_bytes);
        vnew = ld8<0>(qr, hf == 0 ? nvrow + (unsigned)dq * 2u : qkv_bytes);
      }
      float sc[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) sc[j] = 0.f;
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
            sc[j] = __builtin_amdgcn_fdot2_f32_bf16(kp, qp, sc[j], false);
          }
        }
      }
      const bool live = t <= T;
      f4 pl;
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const float v = live ? sc[j] * scale : -__builtin_huge_valf();
        float mm = v;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
        const float nm = fmaxf(mrun[j], mm);  // finite: every chunk has a live position
        const float so = __builtin_amdgcn_exp2f((mrun[j] - nm) * kLog2e);
        const float p = live ? __builtin_amdgcn_exp2f((v - nm) * kLog2e) : 0.f;
        float sm = p;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
        lrun[j] = lrun[j] * so + sm;
        mrun[j] = nm;
        acc[j] *= so;
        pl[j] = p;
      }
      *(f4*)(ps + lane * GRP) = pl;
      __builtin_amdgcn_wave_barrier();
      wait_vm0();  // the value rows are in LDS
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const f4 v = bf16x4_to_f4(*(const U2*)(vs + (32 * hf + r) * HD + dq));
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
      __builtin_amdgcn_wave_barrier();  // the LDS reads above before the next chunk's loads
    }
    if (tail) {
      // The new position (a chunk of one): lane l scores dimensions 2l and
      // 2l + 1, the wave adds the 64 partial sums, and the running softmax
      // takes the one score.  Every load of the wave is complete here.
      wait_vm0();
      __builtin_amdgcn_wave_barrier();
      const bf16x2 kp = *(const bf16x2*)(nk + 2 * lane);
      const f4 vn = bf16x4_to_f4(*(const U2*)(nv + dq));
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        float sj = __builtin_amdgcn_fdot2_f32_bf16(kp, *(const bf16x2*)(qs + j * HD + 2 * lane), 0.f, false);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sj += __shfl_xor(sj, o);
        const float v = sj * scale;
        const float nm = fmaxf(mrun[j], v);
        const float so = __builtin_amdgcn_exp2f((mrun[j] - nm) * kLog2e);
        const float pn = __builtin_amdgcn_exp2f((v - nm) * kLog2e);
        lrun[j] = lrun[j] * so + pn;
        mrun[j] = nm;
        acc[j] *= so;
        if (hf == 0) acc[j] += pn * vn;
      }
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] += __shfl_xor(acc[j][e], 32);
    // The wave's result into its value-row LDS: per head RL floats.
    float* res = (float*)vs;
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (hf == 0) *(f4*)(res + j * RL + dq) = acc[j];
      if (lane == 0) {
        res[j * RL + HD] = mrun[j];
        res[j * RL + HD + 1] = lrun[j];
      }
    }
    __syncthreads();
    // Waves 0..GRP-1, head j = wave: the waves' results added in wave order
    // (lane: dimensions 2 lane, 2 lane + 1), giving the slice's max, sum and
    // accumulator.
    const int j = wave;
    float gm = -__builtin_huge_valf(), L = 0.f, o0 = 0.f, o1 = 0.f;
    if (wave < GRP) {
      for (int w = 0; w < nwv; ++w) gm = fmaxf(gm, ((const float*)(wave_lds(w) + vs_off))[j * RL + HD]);
      for (int w = 0; w < nwv; ++w) {
        const float* rw = (const float*)(wave_lds(w) + vs_off) + j * RL;
        const float f = __builtin_amdgcn_exp2f((rw[HD] - gm) * kLog2e);  // zero for a wave without chunks
        L += rw[HD + 1] * f;
        o0 += rw[2 * lane] * f;
        o1 += rw[2 * lane + 1] * f;
      }
    }
    const unsigned oc = ((unsigned)m * qcols + (unsigned)(g * GRP + j) * HD + 2u * lane) * 2u;
    if (S == 1) {
      if (wave < GRP) {
        const unsigned pk = (unsigned)bf16_bits(o0 / L) | ((unsigned)bf16_bits(o1 / L) << 16);
        __builtin_amdgcn_raw_buffer_store_b32(pk, orr, (int)oc, 0, kAuxNt);
      }
    } else {
      // The slice's result to memory, then the arrival: the XCD-local
      // split-K protocol (all slices of (m, g) run on this XCD).
      const unsigned pbase = (unsigned)(((size_t)m * Hkv + g) * S * GRP * RL);
      if (wave < GRP) {
        const unsigned e = pbase + (unsigned)(sl * GRP + j) * RL;
        st_f32<0>(pr, (e + 2 * lane) * 4u, o0);
        st_f32<0>(pr, (e + 2 * lane + 1) * 4u, o1);
        if (lane == 0) {
          st_f32<0>(pr, (e + HD) * 4u, gm);
          st_f32<0>(pr, (e + HD + 1) * 4u, L);
        }
      }
      splitk_release(SYNC_XCD);
      __syncthreads();
      __shared__ int sh_own;
      if (threadIdx.x < 64) {
        unsigned* ctr = a.actr + m * Hkv + g;
        const unsigned old = splitk_bump(ctr, lane);
        const bool own = splitk_own(ctr, old, S, SYNC_XCD, lane);
        if (lane == 0) sh_own = own ? 1 : 0;
      }
      __syncthreads();
      if (sh_own && wave < GRP) {
        // The S slices' results in slice order; lane s < S holds slice s's max.
        const unsigned ej = pbase + (unsigned)j * RL;
        const float ms = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                             pr, (int)(lane < S ? (ej + (unsigned)lane * GRP * RL + HD) * 4u : pext), 0, kAuxSc1));
        const float ls = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                             pr, (int)(lane < S ? (ej + (unsigned)lane * GRP * RL + HD + 1) * 4u : pext), 0, kAuxSc1));
        U2 av[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          av[q] = ld8<kAuxSc1>(pr, q < S ? (ej + (unsigned)q * GRP * RL + 2u * lane) * 4u : pext);
        float M2 = lane < S ? ms : -__builtin_huge_valf();
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M2 = fmaxf(M2, __shfl_xor(M2, o));
        const float fs = lane < S ? __builtin_amdgcn_exp2f((ms - M2) * kLog2e) : 0.f;
        float L2 = ls * fs;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) L2 += __shfl_xor(L2, o);
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float fq = __shfl(fs, q);  // zero past S
          t0 += __builtin_bit_cast(float, av[q].x) * fq;
          t1 += __builtin_bit_cast(float, av[q].y) * fq;
        }
        const unsigned pk = (unsigned)bf16_bits(t0 / L2) | ((unsigned)bf16_bits(t1 / L2) << 16);
        __builtin_amdgcn_raw_buffer_store_b32(pk, orr, (int)oc, 0, kAuxNt);
      }
    }
    __syncthreads();  // LDS reuse by the next task
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
