// Large-tile MFMA stage ("lt"): the single GEMM from 49 to 256 rows, where a
// weight byte meets enough rows of X that operand traffic inside the CU, not
// HBM, sets the time of the K-chunked path (kc_device.h): there every wave
// owns a K slice of the whole block tile, so its register tile stays small
// and the m-blocks of a column block each load the block's weights again.
//
// Here a workgroup of four or eight waves owns one output tile of TM = 32 MW
// rows by TN = 16 NW WN columns (an m-block of up to 256 rows) over one K
// split, and the waves split the tile 2 x WN (WN = 2 or 4): wave (wm, wn)
// keeps the MW x NW 16 x 16 accumulators of rows [16 MW wm, 16 MW (wm + 1))
// and columns [16 NW wn, 16 NW (wn + 1)), and feeds every A fragment it reads
// to NW MFMAs (v_mfma_f32_16x16x32_bf16) and every B fragment to MW.
//
// Per 64-wide K step the tile's operand blocks (16 rows of X for A, 16 rows
// of W for B, 64 K values each) are fetched with plain 16-byte loads, two
// per block, so that every load instruction reads eight whole 128-byte
// lines; the fetch runs D steps ahead in registers (buffer-to-LDS loads, and
// loads of 64-byte halves of 16 rows, both measured about 20 GB/s per CU
// here, well below whole-line register loads).  Each step's blocks are then
// written to one of two LDS buffers in a row-swizzled layout, from which the
// waves read their MFMA fragments without bank conflicts, while the other
// buffer is multiplied; one workgroup barrier per step (the K-split,
// multi-stage pipeline of the MI355X low-latency GEMM news item, techniques
// 2 and 3, at the batch sizes where the Fleet reading note reports its
// megakernel falling behind, Limitations and open question 4).  Each weight
// byte is read once per workgroup and each X byte once per column block.
//
// Every item runs the same padded number of steps (a multiple of D); loads
// past the split or past M or N read zeros through the buffer range check,
// so each wave issues the same number of loads per step and the vmcnt
// arithmetic below is exact.  Items are (split, column block, m-block),
// taken round-robin by the XCD's workgroups (kc_device.h), so the m-blocks
// of a block run together and share its weight lines through the XCD's L2.
// With S > 1 each wave's accumulator tile is a split-K tile of its own
// (gemm_device.h protocol).
#pragma once
#include "gemm_device.h"

namespace sg {

template <int MW, int NW, int WAVES, int AUX>
__device__ __forceinline__ void lt_stage(const StageDesc& d, uint16_t* lds, int xcd, int slot, int nslots) {
  constexpr int WN = WAVES / 2;  // waves along the columns (two along the rows)
  constexpr int FA = 2 * MW, FB = WN * NW, F = FA + FB;
  constexpr int LPW = lt_loads_per_wave(MW, NW, WAVES);
  constexpr int D = lt_reg_steps(MW, NW, WAVES);  // steps in flight in registers
  static_assert(LPW * (D - 1) < 64, "vmcnt is 6 bits");
  constexpr int TM = 16 * FA;
  constexpr unsigned WTILE = MW * NW * 256;  // floats of one wave's tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches below
  const int wm = wave & 1, wn = wave >> 1;
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
  const int nit = i0 < i1 ? (i1 - i0 + istep - 1) / istep : 0;
  const int MB = d.mb > 1 ? d.mb : 1;
  const int per_split = d.NB * MB;
  auto split_of = [&](int it) { return it / per_split; };
  auto block_of = [&](int it) { return (it - (it / per_split) * per_split) / MB; };
  auto mblk_of = [&](int it) { return it - (it / MB) * MB; };
  // Split-K tile of this wave in item it (one counter and partial block per wave tile).
  auto tile_of = [&](int it) {
    return (unsigned)((((xcd * d.NB + block_of(it)) * MB + mblk_of(it)) * WAVES) + wave);
  };
  const int xc0 = xcd * d.Nx;
  const int xc1 = min(d.N, xc0 + d.Nx);
  const Rsrc wr = make_rsrc(d.W, d.w_bytes);
  const Rsrc xr = make_rsrc(d.X, d.x_bytes);
  const Rsrc yr = make_rsrc(d.Y, d.y_bytes);
  const Rsrc y2r = make_rsrc(d.Y2, d.y2_bytes);
  const Rsrc pr = make_rsrc(d.part, d.part_bytes);
  const int steps = d.steps;

  // Fetch coordinates of local item fl: its split's first K value, the
  // split's end (0 past the last item: those steps load zeros), and the
  // item's first row (of X) and first column (row of W).  The fetch runs D
  // steps ahead of the multiply and items are a multiple of D steps long, so
  // the D fetches of one unrolled group all fall in one item.
  int c_k0 = 0, c_kend = 0, c_row = 0, c_col = 0;
  auto enter = [&](int fl) {
    const bool live = fl < nit;
    const int it = i0 + fl * istep;
    const int s = live ? split_of(it) : 0;
    c_k0 = s * d.KS;
    c_kend = live ? min(d.K, (s + 1) * d.KS) : 0;
    c_row = TM * (live ? mblk_of(it) : 0);
    c_col = xc0 + (live ? block_of(it) : 0) * d.CB;
  };
  // A step covers 64 K values: fragment block f (16 rows or columns x 64 K
  // values, two MFMA k-halves) is fetched by two loads, load h giving lane l
  // the 16 bytes at chunk l % 8 of row 8 h + l / 8, so that every load
  // instruction reads eight whole 128-byte lines.  Load u = WAVES q + wave of
  // the step is (block u / 2, half u % 2); u >= 2 F is padding that reads zeros
  // and is never written.  Operand and offset are selected without a branch,
  // so the compiler keeps exact counts of the loads in flight.
  u4 stg[D][LPW];  // fetched loads of the next D steps
  const int lrow = lane >> 3, lch = lane & 7;
  auto fetch = [&](u4 (&dst)[LPW], int ft) {
    const int k = c_k0 + ft * kLtKStep + 8 * lch;
    const bool kok = k < c_kend;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int u = q * WAVES + wave;  // wave-uniform
      const int f = u >> 1, h = u & 1;
      const bool is_a = f < FA;
      const int row = c_row + 16 * f + 8 * h + lrow;
      const int col = c_col + 16 * (f - FA) + 8 * h + lrow;
      const bool ok = kok && (is_a ? row < d.M : (f < F && col < xc1));
      const unsigned off = is_a ? ((unsigned)row * (unsigned)d.ldx + (unsigned)k) * 2u
                                : ((unsigned)col * (unsigned)d.K + (unsigned)k) * 2u;
      dst[q] = ld16<AUX>(is_a ? xr : wr, ok ? off : (is_a ? d.x_bytes : d.w_bytes));
    }
  };
  // LDS layout of a block: 16 rows of 128 bytes, the chunk c of row r at
  // position c ^ ((r / 2) mod 8), so that the 16 rows one MFMA fragment read
  // takes at the same chunk land in 16 distinct 16-byte bank groups.
  auto swz = [](int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); };
  auto put = [&](const u4 (&src)[LPW], int b) {
    char* const base = (char*)lds + b * (F * 2048);
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int u = q * WAVES + wave;
      const int f = u >> 1, h = u & 1;
      if (f < F) *(u4*)(base + f * 2048 + swz(8 * h + lrow, lch)) = src[q];
    }
  };
  // This lane's fragment offset within a block for k-half kh: row r16,
  // chunk 4 kh + g4 (the MFMA lane order: row or column l % 16, K values
  // 8 (l / 16) .. + 7 of the half).
  const int lo0 = swz(r16, g4), lo1 = swz(r16, 4 + g4);

  f4 acc[MW][NW];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  auto emit = [&](int it) {
    const int m0 = TM * mblk_of(it) + 16 * MW * wm;
    const int c0 = xc0 + block_of(it) * d.CB + 16 * NW * wn + r16;
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 16 * i + 4 * g4 + e;
          const int col = c0 + 16 * j;
          store_out(d, yr, y2r, m < d.M && col < xc1, m, col, acc[i][j][e]);
        }
  };

  // Prologue: steps 0 .. D-1 fetched; step 0 into LDS buffer 0.
  enter(0);
#pragma unroll
  for (int p = 0; p < D; ++p) fetch(stg[p], p);
  wait_vm<LPW * (D - 1)>();
  put(stg[0], 0);
  __syncthreads();
  const char* const ra = (const char*)lds + MW * wm * 2048;          // this wave's A blocks
  const char* const rb = (const char*)lds + (FA + NW * wn) * 2048;   // and B blocks
  for (int li = 0; li < nit; ++li) {
    // The steps of one item (a multiple of D, so every item starts at ring
    // slot 0 and LDS buffer 0): the accumulators stay in the matrix-core
    // registers through this loop; the item's output goes out after it.
    for (int t0 = 0; t0 < steps; t0 += D) {
      // This group's fetches: steps t0 + D .. t0 + 2D - 1 of this item, or
      // the first D steps of the next one.
      int ft = t0 + D;
      if (ft == steps) {
        ft = 0;
        enter(li + 1);
      }
#pragma unroll
      for (int r = 0; r < D; ++r) {
        // Step t0 + r is in LDS buffer r & 1; the next D - 1 steps are in
        // flight in register slots (r + 1) % D .. (r + D - 1) % D.
        const int so = (r & 1) * (F * 2048);
        // Slot r's loads already went to LDS: fetch step t0 + r + D into it.
        fetch(stg[r], ft + r);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int lo = so + (kh ? lo1 : lo0);
          bf16x8 a[MW], b[NW];
#pragma unroll
          for (int i = 0; i < MW; ++i) a[i] = __builtin_bit_cast(bf16x8, *(const u4*)(ra + lo + i * 2048));
#pragma unroll
          for (int j = 0; j < NW; ++j) b[j] = __builtin_bit_cast(bf16x8, *(const u4*)(rb + lo + j * 2048));
#pragma unroll
          for (int i = 0; i < MW; ++i)
#pragma unroll
            for (int j = 0; j < NW; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        // The next step's fragments have arrived once only the D - 1 later
        // steps' loads (and any output stores since) are outstanding; they
        // go to the other LDS buffer, whose last readers (the step before
        // this one) every wave finished before the previous barrier.  The
        // barrier then makes them visible and ends every wave's reads of
        // buffer r & 1.
        wait_vm<LPW * (D - 1)>();
        put(stg[(r + 1) % D], (r + 1) & 1);
        __syncthreads();
      }
    }
    const int it = i0 + li * istep;
    if (d.S == 1) {
      emit(it);
    } else {
      const unsigned base = (tile_of(it) * d.S + split_of(it)) * WTILE;
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) st_f4<0>(pr, (base + (i * NW + j) * 256 + lane * 4) * 4u, acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int j = 0; j < NW; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
  }
  wait_vm0();

  if (d.S > 1 && nit > 0) {
    splitk_release(d.sync);
    for (int c0 = 0; c0 < nit; c0 += 4) {
      unsigned old[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) old[q] = c0 + q < nit ? splitk_bump(d.ctr + tile_of(i0 + (c0 + q) * istep), lane) : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (c0 + q >= nit) break;
        const int itq = i0 + (c0 + q) * istep;
        const unsigned tile = tile_of(itq);
        if (!splitk_own(d.ctr + tile, old[q], d.S, d.sync, lane)) continue;
        // Partial layout of a wave tile: fragment (i, j) at (i NW + j) x 256
        // floats, the [MW][NW] order sum_partials_f4 reads.
#pragma unroll
        for (int i = 0; i < MW; ++i)
#pragma unroll
          for (int j = 0; j < NW; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
        if (d.sync == SYNC_XCD) {
          sum_partials_f4<kAuxSc1, MW, NW>(pr, tile * d.S * WTILE, WTILE, d.S, lane, acc, d.part_bytes);
        } else {
          sum_partials_f4<0, MW, NW>(pr, tile * d.S * WTILE, WTILE, d.S, lane, acc, d.part_bytes);
        }
        emit(itq);
      }
    }
  }
}

}  // namespace sg
