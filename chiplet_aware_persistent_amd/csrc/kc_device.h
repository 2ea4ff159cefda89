// K-chunked MFMA stage ("kc"): the MFMA path for larger M, where the rows of
// X over a whole K split no longer fit the LDS next to anything else.
//
// The eight waves of a workgroup work on one item at a time: a block of NTW
// 16-column weight tiles over one K split (paired: NTW/2 gate tiles and the
// NTW/2 matching up tiles).  The split is walked in chunks of 512 K values;
// in chunk c wave w streams k-step 8c + w (64 K values) of all NTW tiles, so
// the workgroup reads each weight byte once and every wave keeps an fp32
// accumulator per tile and m-tile across the whole split.  One A fragment
// read from LDS feeds NTW tiles' MFMAs, a factor NTW fewer LDS reads per
// weight byte than one tile per wave.
//
// X goes through LDS one chunk at a time, double-buffered: while the waves
// multiply chunk c out of one buffer, the buffer-to-LDS loads of chunk c + 1
// fill the other.  A split's X window therefore no longer has to fit the LDS
// at once, so the planner is free to take few (or no) K splits at M = 64 and
// keep the split-K partials, their HBM round trip and their finalize tails
// small (the K-chunked, multi-stage LDS pipeline of the MI355X low-latency
// GEMM news item, techniques 2 and 3; the Fleet reading note names the
// missing wave-level K split as why its megakernel falls behind at batch 64,
// Limitations and open question 4).
//
// Beyond 64 rows (M up to 256) an item also names an m-block of 64 rows: the
// items of one (split, column block) are its m-blocks, m-block fastest, and
// the workgroups of an XCD take the items round-robin (workgroup w: items w,
// w + 32, ...), so the m-blocks of a column block run at the same time on
// neighbouring workgroups of one XCD and its weight lines are fetched from
// HBM once and read from that XCD's L2 by the others: the M-major window of
// the Fleet reading note (section 3f, Eq.(1): with R = 4 concurrent readers
// of a line, a weight hit rate of 1 - 1/R), here at T_M = 64.
//
// At the end of an item the eight per-wave sums are added through LDS in a
// fixed tree order (w + w+4, then + w+2, then + w+1), so the result does not
// depend on timing; wave 0 then writes Y (or, with S > 1, the split's
// partial, added up by the split-K owner in split order as in gemm_device.h).
#pragma once
#include "gemm_device.h"

namespace sg {

constexpr int kKcWaves = 8;                          // waves per workgroup, all on one item
constexpr int kKcChunk = kKcWaves * kMfmaKStep;      // K values per chunk: one k-step per wave
constexpr int kKcRow = kKcChunk + 8;                 // LDS row stride of an X chunk (elements)

// Weight steps (chunks) in flight per wave: NTW tiles x 2 loads per step.
// Inside the layer chain, four m-tiles keep one step: the chain's own state
// and four m-tiles' accumulators leave no registers for a second.
constexpr int kc_ring_depth(int ntw, int mt, bool chain) {
  return (chain && mt >= 4) || ntw >= 6 ? 1 : (ntw >= 4 ? 2 : 4);
}

// X chunk: rows [m0, m0 + mrows) x K values [k0, k0 + kKcChunk) of X into an
// LDS buffer of xbuf bytes (buffer row r = X row m0 + r, row stride kKcRow),
// zero outside those rows and [k0, kend) (so buffer row mrows, when the
// buffer has it, is a zero row).  One wave instruction fills one kilobyte;
// the waves take the kilobytes in turn.  With kend <= k0 the whole buffer is
// written with zeros (the loads are still issued, so every wave issues the
// same number of loads per step).
__device__ __forceinline__ void stage_x_chunk(const StageDesc& d, uint16_t* buf, int k0, int kend, Rsrc xr,
                                              int m0 = 0, int mrows = 1 << 30) {
  const int lane = threadIdx.x & 63;
  const int pieces = d.xbuf >> 10;
  const int rows_ok = min(mrows, d.M - m0);
  for (int c = (int)(threadIdx.x >> 6); c < pieces; c += kKcWaves) {
    const int e = (c * 1024 + lane * 16) >> 1;
    const int row = e / kKcRow;
    const int col = e - row * kKcRow;
    const int k = k0 + col;
    const bool valid = row < rows_ok && col < kKcChunk && k < kend;
    const unsigned off = valid ? ((unsigned)(m0 + row) * (unsigned)d.ldx + (unsigned)k) * 2u : d.x_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)((char*)buf + c * 1024),
                                             16, off, 0, 0, 0);
  }
}

// Items: (split s, block b, m-block q), split-major, m-block fastest (d.mb
// m-blocks of 16 MT rows; one when every row fits one item).  Workgroup slot
// w of nslots takes the contiguous range [first_item_of_wg(w),
// first_item_of_wg(w + 1)), or with d.rr the items w, w + nslots, ...  Block
// b of XCD x covers the output columns [x*Nx + b*CB, x*Nx + (b+1)*CB), CB =
// 16 NTW (paired: 16 NTW/2, with the up rows pair_off rows further on).
// d.steps is the number of chunks per item (a multiple of the ring depth).
template <int MT, int NTW, bool PAIRED, int AUX, typename Hook = NoHook, bool CHAIN = false>
__device__ __forceinline__ bool mfma_kc_stage(const StageDesc& d, uint16_t* xs, int xcd, int slot, int nslots,
                              Hook pre_x = Hook()) {
  constexpr int P = kc_ring_depth(NTW, MT, CHAIN);
  static_assert(!PAIRED || NTW % 2 == 0, "a paired block holds whole (gate, up) tile pairs");
  constexpr int NP = PAIRED ? NTW / 2 : NTW;  // 16-column output tiles of a block
  constexpr unsigned TILE = NTW * MT * 256;   // floats of one item's partial
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;          // this wave's k-step within each chunk
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  int i0, i1, istep = 1;
  if (d.rr) {
    i0 = slot;
    i1 = d.items;
    istep = nslots;
  } else {
    i0 = first_item_of_wg(d.items, slot, nslots);
    i1 = first_item_of_wg(d.items, slot + 1, nslots);
  }
  const int nit = i0 < i1 ? (i1 - i0 + istep - 1) / istep : 0;  // items of this workgroup
  const int nc = d.steps;
  const int MB = d.mb > 1 ? d.mb : 1;
  constexpr int TM = 16 * MT;  // rows of an m-block
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const Rsrc pr = make_rsrc(d.part, d.part_bytes);
  const int per_split = d.NB * MB;
  auto split_of = [&](int it) { return it / per_split; };
  auto block_of = [&](int it) { return (it - (it / per_split) * per_split) / MB; };
  auto mblk_of = [&](int it) { return it - (it / MB) * MB; };
  // Split-K tile (counter and partial block) of item it.
  auto tile_of = [&](int it) { return (unsigned)((xcd * d.NB + block_of(it)) * MB + mblk_of(it)); };
  auto xbuf = [&](int b) { return (uint16_t*)((char*)xs + b * d.xbuf); };

  // Weight stream: the full-line load layout of the MFMA path (load h gives
  // lane l the 16-byte chunk (l%8)^4h of row 8h + l/8 of a tile), permuted
  // into the B operand by ds_bpermute.
  struct Src {
    unsigned base;  // byte offset of (row col0, k0)
    int klim;       // K values of the item's split
    int col0;       // first output column of the block
  };
  const int lr8 = lane >> 3;
  int lch[2];
  unsigned loff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    lch[h] = (lane & 7) ^ (4 * h);
    loff[h] = ((unsigned)(8 * h + lr8) * (unsigned)d.K + 8u * (unsigned)lch[h]) * 2u;
  }
  auto src_of = [&](int it) -> Src {
    Src r;
    if (it >= i1) { r.base = 0; r.klim = 0; r.col0 = xc1; return r; }
    const int s_ = split_of(it);
    const int k0 = s_ * d.KS;
    const int col0 = xc0 + block_of(it) * d.CB;
    r.base = ((unsigned)col0 * (unsigned)d.K + (unsigned)k0) * 2u;
    r.klim = min(d.K, k0 + d.KS) - k0;
    r.col0 = col0;
    return r;
  };
  // Weight row offset (bytes) of tile j from row col0.
  auto jrow = [&](int j) -> unsigned {
    if (PAIRED && j >= NP) return ((unsigned)d.pair_off + 16u * (unsigned)(j - NP)) * (unsigned)d.K * 2u;
    return 16u * (unsigned)j * (unsigned)d.K * 2u;
  };
  // Step t of an item: k-step 8t + wave.  Masked lanes read past the extent
  // (zeros); issue is branch-free, so the compiler keeps exact load counts.
  auto issue_tile = [&](u4(&dst)[2], const Src& sr, int t, int j) {
    const int ks = t * kKcWaves + wave;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = sr.col0 + 16 * (PAIRED ? j % NP : j) + 8 * h + lr8;
      const bool valid = col < xc1 && ks * kMfmaKStep + 8 * lch[h] < sr.klim;
      const unsigned off = sr.base + loff[h] + jrow(j) + (unsigned)ks * (kMfmaKStep * 2u);
      dst[h] = ld16<AUX>(wr, valid ? off : d.w_bytes);
    }
  };
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
  auto emit = [&](int col0, int m0, const f4 (&v)[NTW][MT]) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int col = col0 + 16 * j + r16;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 16 * i + 4 * g4 + e;
          const bool ok = m < d.M && col < xc1;
          if constexpr (PAIRED) {
            store_out(d, yr, y2r, ok, m, col, silu_mul(v[j][i][e], v[j + NP][i][e]));
          } else {
            store_out(d, yr, y2r, ok, m, col, v[j][i][e]);
          }
        }
    }
  };
  // K range and first row of item it.
  int k0, kend, m0;
  auto item_k = [&](int it) {
    k0 = split_of(it) * d.KS;
    kend = min(d.K, k0 + d.KS);
    m0 = TM * mblk_of(it);
  };

  // A-operand rows: m-tile i, lane row 16i + r16 of the item's m-block, or
  // the buffer's zero row (row min(TM, M - m0)) past M.
  int xro[MT];
  auto set_rows = [&]() {
#pragma unroll
    for (int i = 0; i < MT; ++i) xro[i] = min(16 * i + r16, d.M - m0) * kKcRow;
  };
  bf16x8 xa[2][MT];

  constexpr bool early = __is_same(Hook, NoHook);
  item_k(i0 < i1 ? i0 : 0);
  if (i0 >= i1) kend = 0;
  set_rows();
  if constexpr (early) stage_x_chunk(d, xbuf(0), k0, kend, xr, m0, TM);
  u4 ring[P][NTW][2];
  Src sc = src_of(i0), sn = src_of(i0 + istep);
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int j = 0; j < NTW; ++j) issue_tile(ring[p][j], sc, p, j);
  if (!pre_x()) return false;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (early) {
    wait_vm<P * NTW * 2>();
  } else {
    stage_x_chunk(d, xbuf(0), k0, kend, xr, m0, TM);
    wait_vm0();
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  f4 acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = f4{0.f, 0.f, 0.f, 0.f};
  f4* red = (f4*)xs;
  int it = i0, t0 = 0;
  const int total = nit * nc;
  for (int T = 0; T < total; T += P) {
    const bool here = t0 + P < nc;  // this group's refills stay in the item
    Src sr;
    sr.base = here ? sc.base : sn.base;
    sr.klim = here ? sc.klim : sn.klim;
    sr.col0 = here ? sc.col0 : sn.col0;
    const int tn = here ? t0 + P : t0 + P - nc;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int t = t0 + p;
      // Chunk t + 1 of this item into the other buffer (zeros after the last).
      stage_x_chunk(d, xbuf((t + 1) & 1), k0 + (t + 1) * kKcChunk, t + 1 < nc ? kend : 0, xr, m0, TM);
      const uint16_t* xb = xbuf(t & 1) + wave * kMfmaKStep + 8 * g4;
      // Both halves' A fragments first; then tile by tile, both halves and
      // the tile's reload right behind them, so each tile waits only for its
      // own loads and the wave keeps the rest of the ring in flight.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < MT; ++i) xa[h][i] = __builtin_bit_cast(bf16x8, *(const u4*)(xb + xro[i] + 32 * h));
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 wb = to_b(ring[p][j], h);
#pragma unroll
          for (int i = 0; i < MT; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[h][i], wb, acc[j][i], 0, 0, 0);
        }
        issue_tile(ring[p][j], sr, tn + p, j);
        __builtin_amdgcn_sched_barrier(0);  // the reload right behind its last use
      }
      // Only this step's refills may still be outstanding: chunk t + 1 is in
      // LDS for this wave's kilobytes; the barrier makes it whole, and frees
      // buffer t & 1 for chunk t + 2.
      wait_vm<NTW * 2>();
      __syncthreads();
    }
    t0 += P;
    if (t0 == nc) {  // item complete: add the eight waves' sums in tree order
#pragma unroll
      for (int r = kKcWaves / 2; r >= 1; r >>= 1) {
        if (wave >= r && wave < 2 * r) {
#pragma unroll
          for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i) red[(((wave - r) * NTW + j) * MT + i) * 64 + lane] = acc[j][i];
        }
        __syncthreads();
        if (wave < r) {
#pragma unroll
          for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[j][i] += red[((wave * NTW + j) * MT + i) * 64 + lane];
        }
        __syncthreads();
      }
      if (wave == 0) {
        if (d.S == 1) {
          emit(xc0 + block_of(it) * d.CB, m0, acc);
        } else {
          const unsigned base = (tile_of(it) * d.S + split_of(it)) * TILE;
#pragma unroll
          for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int i = 0; i < MT; ++i)
              st_f4<0>(pr, (base + (j * MT + i) * 256 + lane * 4) * 4u, acc[j][i]);
        }
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[j][i] = f4{0.f, 0.f, 0.f, 0.f};
      it += istep;
      t0 = 0;
      sc = sn;
      sn = src_of(it + istep);
      if (it < i1) {
        // The next item's first chunk: the reduction used the buffers, so
        // its X is loaded only now, and waiting for it also waits for the
        // weights already in flight.
        item_k(it);
        set_rows();
        stage_x_chunk(d, xbuf(0), k0, kend, xr, m0, TM);
        wait_vm0();
        __syncthreads();
      }
    }
  }

  if (d.S > 1 && nit > 0 && wave == 0) {
    splitk_release(d.sync);
    for (int c0 = 0; c0 < nit; c0 += 4) {
      unsigned old[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        old[q] = c0 + q < nit ? splitk_bump(d.ctr + tile_of(i0 + (c0 + q) * istep), lane) : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (c0 + q >= nit) break;
        const int itq = i0 + (c0 + q) * istep;
        const unsigned tile = tile_of(itq);
        if (!splitk_own(d.ctr + tile, old[q], d.S, d.sync, lane)) continue;
        f4 tot[NTW][MT];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int i = 0; i < MT; ++i) tot[j][i] = f4{0.f, 0.f, 0.f, 0.f};
        if (d.sync == SYNC_XCD) {
          sum_partials_f4<kAuxSc1, NTW, MT>(pr, tile * d.S * TILE, TILE, d.S, lane, tot, d.part_bytes);
        } else {
          sum_partials_f4<0, NTW, MT>(pr, tile * d.S * TILE, TILE, d.S, lane, tot, d.part_bytes);
        }
        emit(xc0 + block_of(itq) * d.CB, TM * mblk_of(itq), tot);
      }
    }
  }
  return true;
}

}  // namespace sg
