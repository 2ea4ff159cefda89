// C ABI of libsgemm.so: validation, planning and launches.  See include/sgemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "../../include/sgemm.h"
#include "launch.h"
#include "stage_desc.h"

using namespace sg;

namespace {

constexpr size_t kCtl = 256;            // control block: status word, done counter, slot claims
constexpr int kLdsCu = 160 * 1024;      // LDS of one CU (one workgroup per CU)
// Static LDS a kernel may declare besides the planned dynamic region (the
// chain's two flags take 16 bytes); the build refuses a kernel with more.
constexpr int kStaticLdsReserve = 256;
constexpr int kLdsMax = kLdsCu - kStaticLdsReserve;  // dynamic LDS budget of a plan
constexpr size_t kMaxOperand = (size_t)1 << 31;  // buffer extents are 31-bit here
constexpr int kWgPerXcd = 32;           // one workgroup per CU, 32 CUs per XCD
constexpr int kMaxM = 256;              // single GEMM rows (chain and decoder: 64)

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Decomposition of one GEMM stage (see gemm_device.h for how it is executed).
struct Geo {
  int path = 0;        // 0 dot2, 1 MFMA, 2 MFMA m-tile items, 3 K-chunked MFMA
  int M = 0, K = 0, N = 0;
  int ta = 0, tb = 0;  // template parameters: dot2 (M, G); MFMA (MT, NT)
  int waves = 8, wpi = 8, ng = 1, TN = 0, CB = 0, Nx = 0, NB = 0, S = 1, KS = 0, steps = 0, items = 0;
  int ksl = 1, kss = 0;
  int win = 0, xrow = 0, lds = 0, red_off = 0, stash_off = 0, stash_cap = 0;
  int paired = 0, pair_off = 0;
  int ring = 0;    // ring depth (k-steps in flight per wave)
  int mtiles = 1;  // m-tile items (ablation): items per (split, column block), m-tile fastest
  int slots = 32;  // workgroups per XCD that share the items (31 with a scheduler workgroup)
  int xbuf = 0;    // K-chunked path: bytes of one X chunk buffer
  int nfast = 0;   // m-tile items in the M-split order (column block fastest)
  int kc_chain = 0;  // K-chunked path: a stage of the layer chain (its ring depth rule)
  int mb = 1;        // K-chunked path: m-blocks of 16 ta rows per (split, column block), M > 64
  int rr = 0;        // dot2 path, S = 1: items round-robin over the XCD's streams
  int wpf = 0, wpf_off = 0;  // chain dot2 stage: first-item steps whose weights go to LDS before the wait
  size_t ctr_count = 0, part_floats = 0;
  double est_us = 0.0;
};

// Integer from the environment: dflt when unset or empty; false when the
// value is not a whole decimal integer.
bool env_int(const char* name, int dflt, int* out) {
  const char* v = std::getenv(name);
  if (!v || !*v) {
    *out = dflt;
    return true;
  }
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  if (*end != '\0' || x < -(1L << 30) || x > (1L << 30)) return false;
  *out = (int)x;
  return true;
}

// Cost-model constants of one launch context (a single GEMM launch, or a
// stage inside the persistent chain, where X comes from other XCDs' fresh
// writes and the neighbouring stages overlap the tails).
struct Cost {
  double alpha;      // how far one item stream may exceed its 1/ng share of the CU
  double x_bw;       // X staging rate per CU, bytes/s
  double split_us;   // split-K arrival and finalize round trip
  double fin_us_kb;  // per kilobyte of partials an owner reads
  double ksl_us;     // per item with K slices (two workgroup barriers, LDS exchange)
  bool chain;        // a chain stage (up to two m-tiles it keeps the deeper MFMA ring)
  int lds_reserve = 0;  // LDS bytes kept free after the stage's own (the decoder's norm factors)
};
constexpr Cost kCostGemm{1.0, 200.0e9, 6.0, 0.05, 0.0, false};
// Chain constants fitted to whole-chain times of per-stage forced plans at
// M = 1..64 (36 layers, d = q = 4096, d_ff = 12288): X comes from other XCDs'
// fresh writes (slower than a warm window), while a split's finalize overlaps
// the neighbouring stages' streams.
constexpr Cost kCostChain{1.25, 75.0e9, 0.5, 0.05, 0.25, true};

// Fill the derived fields of g for (path, template params, waves, wpi, ksl,
// S); returns false when the candidate does not fit (LDS, instantiations).
bool shape_geo(Geo& g, int want_S, const Cost& cost) {
  const int kstep = g.path == 0 ? kDot2KStep : kMfmaKStep;
  if (g.wpi % g.ksl) return false;
  // Output columns per wave: dot2 G (paired: G/2 gate/up pairs), MFMA 16 per n-tile.
  if (g.path == 0 && g.paired && g.tb % 2) return false;
  g.TN = g.path == 0 ? (g.paired ? g.tb / 2 : g.tb) : (g.paired ? 16 : 16 * g.tb);
  g.ng = g.waves / g.wpi;
  if (g.ksl > 1 && g.ng != 1) return false;  // K slices reduce with workgroup barriers
  g.CB = g.wpi / g.ksl * g.TN;
  g.Nx = (int)round_up((size_t)ceil_div(g.N, kXcds), 16);
  g.NB = ceil_div(g.Nx, g.CB);
  // Splits start on whole 128-byte lines of the weight rows (64 values), so
  // no line is fetched by two splits.
  g.KS = (int)round_up((size_t)ceil_div(g.K, want_S), 64);
  g.S = ceil_div(g.K, g.KS);
  g.kss = g.ksl > 1 ? (int)round_up((size_t)ceil_div(g.KS, g.ksl), kstep) : g.KS;
  if (g.ksl > 1 && (g.ksl - 1) * g.kss >= g.KS) return false;  // an empty slice
  const int ring = g.path == 0 ? ring_depth_dot2(g.tb)
                                : ring_depth_mfma(g.paired ? 2 : g.tb, cost.chain && g.ta <= 2);
  const int pad = g.path == 0 ? ring : step_pad_mfma(g.paired ? 2 : g.tb);
  g.steps = ceil_div(ceil_div(g.kss, kstep), pad) * pad;  // a multiple of the ring depth
  g.ring = ring;
  g.items = g.NB * g.S * g.mtiles;
  // A workgroup stages X once for all splits its contiguous item range
  // touches: the window is (span - 1) splits plus the last slice's padded steps.
  const int per_split = g.NB * g.mtiles;
  int span = 1;
  for (int w = 0; w < g.slots; ++w) {
    const int i0 = (int)((long long)g.items * w / g.slots);
    const int i1 = (int)((long long)g.items * (w + 1) / g.slots);
    if (i0 < i1) span = std::max(span, (i1 - 1) / per_split - i0 / per_split + 1);
  }
  g.win = (span - 1) * g.KS + (g.ksl - 1) * g.kss + g.steps * kstep;
  g.win = (int)round_up((size_t)g.win, 8);
  // MFMA: the rows of X plus one zero row when the M-tiles overhang M.
  const int rows = g.path == 0 ? g.M : std::min(16 * g.ta * g.mtiles, g.M + 1);
  g.xrow = g.path == 0 ? g.win : g.win + 8;
  // LDS: X window, K-slice reduction buffer, output stash.
  const int tile_bytes = g.path == 0 ? 64 * 4 : g.tb * g.ta * 1024;  // one wave's item result
  g.red_off = (int)round_up((size_t)rows * g.xrow * 2, 1024);  // X is staged in 1 KB chunks
  const int red_bytes = g.ksl > 1 ? (g.wpi / g.ksl) * (g.ksl - 1) * tile_bytes : 0;
  g.stash_off = g.red_off + red_bytes;
  const int owners = g.ksl > 1 ? g.wpi / g.ksl : g.waves;
  const int per_stream = ceil_div(g.items, g.slots * g.ng);
  const int lds_cap = kLdsMax - cost.lds_reserve;
  g.stash_cap = std::max(0, std::min(per_stream, (lds_cap - g.stash_off) / (owners * tile_bytes)));
  g.lds = g.stash_off + owners * g.stash_cap * tile_bytes;
  const int vals = g.path == 0 ? g.tb * g.M : g.tb * g.ta * 256;
  g.ctr_count = (size_t)kXcds * g.NB * g.wpi * g.mtiles;
  g.part_floats = g.S > 1 ? g.ctr_count * (size_t)g.S * vals : 0;
  if (g.stash_off > lds_cap) return false;
  // MFMA with S == 1 emits Y only from the stash (no epilogue inside the
  // weight loop), so every item of a stream must fit it.
  if (g.path == 1 && g.S == 1 && g.stash_cap < per_stream) return false;
  if (!gemm_variant_exists(g.path, g.ta, g.tb) && !g.paired) return false;
  // Cost model (microseconds): streaming time of the busiest workgroup at the
  // per-CU share of HBM bandwidth, its X staging, per-item costs (a store at
  // item end, K-slice barriers), and for split-K the finalize round trips
  // (arrival atomics, partial reads) at the end.  A workgroup keeps waves *
  // 16 KB of weight loads in flight; fewer than 8 waves leave the per-CU share
  // unreached, and so do ring slots spent on padded steps.  The constants
  // were fitted to kernel durations of forced plans over the decode shapes
  // (the planner's pick is within 1.5% of the fastest measured plan on
  // average).
  // Per-CU rates (bytes of W per second): the HBM share, the LDS traffic the
  // inner loop generates per weight byte (dot2: X reads M/G; MFMA: A reads
  // MT/NT plus the B permute), and dot2's VALU time (4 M dot2 cycles per KB
  // per SIMD quartet, on top of the loop overhead).
  double bw_cu = 8.0e12 * 0.85 / 256.0 * (g.waves >= 8 ? 1.0 : 0.6);
  const double lds_cu = 128.0 * 2.4e9 * 0.5;
  const double lds_per_w = g.path == 0 ? (double)g.M / g.tb : (double)g.ta / g.tb + 1.0;
  bw_cu = std::min(bw_cu, lds_cu / lds_per_w);
  if (g.path == 0) bw_cu = std::min(bw_cu, 1024.0 / (4.0 * g.M + 4.0) * 2.4e9 * 0.7);
  const double item_bytes = (double)g.CB * g.KS * 2.0 * (g.paired ? 2.0 : 1.0);
  const double slot_bytes = (double)g.CB * g.steps * kstep * g.ksl * 2.0 * (g.paired ? 2.0 : 1.0);
  bw_cu *= item_bytes / slot_bytes;
  const double part_bytes = g.S > 1 ? (double)g.CB * g.M * 4.0 * 2.0 * (g.paired ? 2.0 : 1.0) : 0.0;
  // The busiest workgroup's bytes, or its busiest stream's at alpha times
  // the stream's fair share of the CU if that is longer.  Alpha is 1 for a
  // single launch; inside the chain the neighbouring stages keep HBM busy and
  // unevenly loaded waves cost less.
  const double wg_items = ceil_div(g.items, g.slots);
  const double wg_bytes = std::max(wg_items * (item_bytes + part_bytes),
                                   (double)g.ng * per_stream * (item_bytes + part_bytes) / cost.alpha);
  const double x_us = (double)rows * g.win * 2.0 / cost.x_bw * 1e6;
  const double item_us = (per_stream > g.stash_cap ? 0.1 : 0.05) + (g.ksl > 1 ? cost.ksl_us : 0.0);
  // split-K finalize: arrival round trips plus the owner's partial reads
  // (S tiles of tile_bytes; a dot2 owner lane reads S floats).
  const double fin_kb = g.S * (g.path == 0 ? 0.25 : tile_bytes / 1024.0);
  g.est_us = wg_bytes / bw_cu * 1e6 + per_stream * item_us + x_us +
             (g.S > 1 ? cost.split_us + cost.fin_us_kb * fin_kb : 0.0) +
             (span > 1 ? 0.5 : 0.0);
  return true;
}

bool plan_geo(Geo& best, int M, int K, int N, int path, int paired, int tn_o, int s_o, int waves_o,
              int ksl_o, const Cost& cost, int wpi_o = 0, int mti_rows = 0, int slots = kWgPerXcd) {
  bool found = false;
  const int waves_opts[2] = {8, 4};
  for (int wi = 0; wi < 2; ++wi) {
    const int waves = waves_opts[wi];
    if (waves_o && waves != waves_o) continue;
    for (int wpi = 1; wpi <= waves; wpi *= 2)
    for (int ksl = 1; ksl <= (path == 1 ? wpi : 1); ksl *= 2)
    for (int tb = 1; tb <= 8; ++tb) {
      if (ksl_o && ksl != ksl_o) continue;
      if (wpi_o && wpi != wpi_o) continue;
      Geo g;
      g.path = path; g.M = M; g.K = K; g.N = N; g.waves = waves; g.wpi = wpi; g.ksl = ksl;
      g.paired = paired;
      g.slots = slots;
      if (path == 0) {
        if (tb == 5 || tb == 6 || tb == 7) continue;
        if (tn_o && tb != tn_o) continue;
        g.ta = M; g.tb = tb;
      } else {
        if (tb > 2) continue;
        if (paired && tb != 2) continue;
        if (tn_o && !paired && 16 * tb != tn_o) continue;
        g.ta = (M + 15) / 16; g.tb = tb;
        if (mti_rows) {  // one window of mti_rows rows (16, 32 or 64) per item, one wave per item
          if (wpi != 1 || ksl != 1) continue;
          g.ta = mti_rows / 16;
          g.mtiles = (M + mti_rows - 1) / mti_rows;
          if (!gemm_variant_exists(2, g.ta, g.tb)) continue;
        }
      }
      // The model was fitted up to 16 splits.  With 31 worker slots a
      // workgroup's items straddle two splits, which doubles its X window;
      // up to 32 splits keep it inside the LDS at M = 64 and K = 12288.
      const int s_lo = s_o ? s_o : 1, s_hi = s_o ? s_o : (slots < kWgPerXcd ? 32 : 16);
      for (int s = s_lo; s <= s_hi; ++s) {
        if (s > 1 && (K + s - 1) / s < 8) break;
        Geo c = g;
        if (!shape_geo(c, s, cost)) continue;
        if (c.S != s && !s_o) continue;  // rounding collapsed it to another count
        if (!found || c.est_us < best.est_us - 1e-9) { best = c; found = true; }
      }
    }
  }
  return found;
}

// K-chunked MFMA path (kc_device.h): all eight waves of a workgroup work on
// one item of NTW 16-column tiles over a K split, walking it in 512-wide K
// chunks double-buffered through LDS.  Fill g for (MT, NTW, paired, S); false
// when it does not fit.
constexpr int kKcChunkK = 512;  // K values per chunk (8 waves x one 64-wide k-step)

// Chain and decoder stages with one K split take their items round-robin
// over the XCD's streams (as single launches do): MFMA stages, and dot2
// stages whose waves hold at most 16 (column, row) sums, the kernel's limit
// (gemm_device.h, kRrChainMaxMG); SGEMM_CHAIN_RR=0 keeps contiguous ranges.
// Measured on the 36-layer chain: 1.7% faster at M = 1, 1.3% at M = 2,
// bitwise the same.
bool set_chain_rr(Geo* cg, int n, bool scheduler) {
  int rr = 1;
  if (!env_int("SGEMM_CHAIN_RR", 1, &rr)) return false;
  for (int s = 0; s < n; ++s) {
    Geo& g = cg[s];
    const bool fits = g.path == 0 ? g.M * g.tb <= 16 : (g.path == 1 && g.mtiles == 1);
    g.rr = rr && fits && g.S == 1 && g.wpf == 0 && !scheduler ? 1 : 0;
  }
  return true;
}

// Same rule as the kernel's ring depth (kc_device.h).
int kc_ring(int ntw, int mt, bool chain) { return (chain && mt >= 4) || ntw >= 6 ? 1 : (ntw >= 4 ? 2 : 4); }

bool kc_geo(Geo& g, int want_S, const Cost& cost) {
  const int MT = g.ta, NTW = g.tb;
  if (g.paired && NTW % 2) return false;
  const int NP = g.paired ? NTW / 2 : NTW;
  const int ring = kc_ring(NTW, MT, g.kc_chain);
  g.waves = 8; g.wpi = 8; g.ng = 1; g.ksl = 1;
  g.TN = 16;
  g.CB = NP * 16;
  g.Nx = (int)round_up((size_t)ceil_div(g.N, kXcds), 16);
  g.NB = ceil_div(g.Nx, g.CB);
  // Splits: whole chunk groups (the chunk count of an item is a multiple of
  // the ring depth, so refills of the last steps fall into the next item).
  g.KS = (int)round_up((size_t)ceil_div(g.K, want_S), (size_t)kKcChunkK * ring);
  g.S = ceil_div(g.K, g.KS);
  g.kss = g.KS;
  g.steps = g.KS / kKcChunkK;  // chunks per item
  g.ring = ring;
  // Beyond 16 MT rows, m-blocks of 16 MT rows: items (split, block, m-block),
  // m-block fastest, taken round-robin so a block's m-blocks run together.
  g.mb = ceil_div(g.M, 16 * MT);
  g.items = g.NB * g.S * g.mb;
  if (g.mb > 1) g.rr = 1;
  g.mtiles = 1;
  // X rows of a chunk buffer: the m-block's, plus the zero row that the
  // A-operand lanes past M read when the last m-block is partial.
  const int rows = std::min(16 * MT, g.M + 1);
  g.win = kKcChunkK;
  g.xrow = kKcChunkK + 8;
  g.xbuf = (int)round_up((size_t)rows * g.xrow * 2, 1024);
  const int red = 4 * NTW * MT * 1024;  // first round of the eight-wave tree
  g.lds = std::max(2 * g.xbuf, red);
  g.red_off = g.lds; g.stash_off = g.lds; g.stash_cap = 0;
  if (g.lds > kLdsMax) return false;
  g.ctr_count = (size_t)kXcds * g.NB * g.mb;
  g.part_floats = g.S > 1 ? g.ctr_count * (size_t)g.S * NTW * MT * 256 : 0;
  // Cost (microseconds): a workgroup's weight bytes at its share of HBM, or
  // its weight plus X bytes at the CU's L2 read rate if that is longer; per
  // item the reduction, the first chunk's X and the ring drain; per chunk a
  // workgroup barrier; for S > 1 the partials' round trip and the finalize.
  // With m-blocks a weight byte comes from HBM once per block (the other
  // m-blocks read it from L2), and the matrix cores' time is added.
  const double wg_items = ceil_div(g.items, g.slots);
  const double w_bytes = wg_items * NTW * 16.0 * g.steps * kKcChunkK * 2.0;
  const double x_bytes = wg_items * rows * g.steps * (double)kKcChunkK * 2.0;
  const double p_bytes = g.S > 1 ? wg_items * NTW * MT * 1024.0 * 2.0 : 0.0;
  const double bw_cu = 8.0e12 * 0.85 / 256.0;
  const double cu_rd = 110.0e9;
  double mfma_us = 0.0;
  if (g.mb > 1) {
    // 16 MT x 16 NTW x KS multiply-adds per item at half the CU's dense
    // bf16 rate (2.5 PFLOP/s over 256 CUs).
    const double flops = wg_items * 2.0 * 16.0 * MT * 16.0 * NTW * g.steps * kKcChunkK;
    mfma_us = flops / (2.5e15 / 256.0 * 0.5) * 1e6;
  }
  g.est_us = std::max(std::max(w_bytes / g.mb / bw_cu, (w_bytes + x_bytes + p_bytes) / cu_rd) * 1e6, mfma_us) +
             wg_items * (1.5 + rows * kKcChunkK * 2.0 / cost.x_bw * 1e6) + wg_items * g.steps * 0.05 +
             (g.S > 1 ? cost.split_us + cost.fin_us_kb * g.S * NTW * MT : 0.0);
  return true;
}

// Large-tile MFMA path (lt_device.h, path 5), single GEMM at M > 64: four
// waves over a workgroup tile of 32 MW rows x 32 NW columns, 32-wide K steps
// through a ring of LDS slots.  Fill g for (MW, NW, S); false when it does
// not fit.
bool lt_geo(Geo& g, int want_S) {
  const int MW = g.ta, NW = g.tb, WV = g.waves;  // WV = 4 or 8 waves (2 x WV/2 over the tile)
  g.path = WV == 8 ? 6 : 5;
  g.wpi = WV; g.ng = 1; g.ksl = 1;
  g.TN = 16;
  g.CB = 16 * NW * (WV / 2);
  g.Nx = (int)round_up((size_t)ceil_div(g.N, kXcds), 16);
  g.NB = ceil_div(g.Nx, g.CB);
  // Splits start on whole 128-byte lines; every item runs the split's steps
  // (the last split's extra steps read zeros).
  g.KS = (int)round_up((size_t)ceil_div(g.K, want_S), 64);
  g.S = ceil_div(g.K, g.KS);
  g.kss = g.KS;
  g.ring = lt_reg_steps(MW, NW, WV);
  g.steps = (int)round_up((size_t)(g.KS / kLtKStep), (size_t)g.ring);  // a multiple of the ring
  g.mb = ceil_div(g.M, 32 * MW);
  g.items = g.NB * g.S * g.mb;
  g.rr = 1;
  g.mtiles = 1;
  g.lds = lt_lds_bytes(MW, NW, WV);
  g.win = 0; g.xrow = 0; g.xbuf = 0;
  g.red_off = g.lds; g.stash_off = g.lds; g.stash_cap = 0;
  if (g.lds > kLdsMax) return false;
  g.ctr_count = (size_t)kXcds * g.NB * g.mb * WV;
  g.part_floats = g.S > 1 ? g.ctr_count * (size_t)g.S * MW * NW * 256 : 0;
  // Cost (microseconds): per workgroup the longest of its weight bytes from
  // HBM (m-blocks of one block share them through L2), its weight and X
  // bytes from L2, and its matrix-core work at 70% of the CU's dense bf16
  // rate; plus a per-step barrier and, with splits, the partials' round
  // trip and the finalize.
  const double wg_items = ceil_div(g.items, g.slots);
  const double ks = (double)g.steps * kLtKStep;
  const double tm = 32.0 * MW, cb = (double)g.CB;
  const double w_bytes = wg_items * cb * ks * 2.0, x_bytes = wg_items * tm * ks * 2.0;
  const double flops = wg_items * 2.0 * tm * cb * ks;
  const double p_bytes = g.S > 1 ? wg_items * tm * cb * 4.0 * 2.0 : 0.0;
  const double bw_cu = 8.0e12 * 0.85 / 256.0, cu_rd = 110.0e9, mfma_cu = 2.5e15 / 256.0 * 0.7;
  g.est_us = std::max(std::max((w_bytes / g.mb + p_bytes) / bw_cu, (w_bytes + x_bytes) / cu_rd), flops / mfma_cu) * 1e6 +
             wg_items * g.steps * 0.02 + (g.S > 1 ? 6.0 : 0.0);
  return true;
}

// tm_o, tn_o, w_o: forced tile rows, tile columns and waves.  Unforced, the
// tile is 128 (or 64, below) x 192 with eight waves, the fastest of the tiles
// measured on every projection shape at M = 128 and 256 (cold HBM: 76.1 us at
// 256 x 4096 x 24576 against 93.8-98.7 us for the four-wave tiles, 111.0
// against 142.8 us at 256 x 7168 x 18432); the cost model then only picks
// the split count.
bool plan_lt(Geo& best, int M, int K, int N, int tm_o, int tn_o, int w_o, int s_o) {
  bool found = false;
  const bool free_tile = !tm_o && !tn_o && !w_o;
  for (int wv : {4, 8}) {
    if (w_o && wv != w_o) continue;
    if (free_tile && wv != 8) continue;
    for (int mw : {2, 4, 8}) {
      if (tm_o && 32 * mw != tm_o) continue;
      // Unforced: 128-row tiles above 128 rows, 64-row ones up to 128 (two
      // m-blocks sharing the weights through L2 instead of K splits or
      // zero rows; measured: 65 x 4096 x 24576 50.4 against 53.2 us,
      // 128 x 7168 x 18432 82.7 against 86.5, 128 x 12288 x 4096 42.5
      // against 44.9, 128 x 4096 x 4096 23.9 against 27.7).
      const int mw_free = M <= 128 ? 2 : 4;
      if (free_tile && mw != mw_free) continue;
      for (int nw : {3, 6}) {
        if (tn_o && 16 * nw * (wv / 2) != tn_o) continue;
        if (free_tile && nw != 3) continue;
        if (!gemm_variant_exists(wv == 8 ? 6 : 5, mw, nw)) continue;
        const int s_lo = s_o ? s_o : 1, s_hi = s_o ? s_o : 8;
        for (int s = s_lo; s <= s_hi; ++s) {
          Geo c;
          c.M = M; c.K = K; c.N = N; c.ta = mw; c.tb = nw; c.waves = wv; c.slots = kWgPerXcd;
          if (!lt_geo(c, s)) continue;
          if (c.S != s && !s_o) continue;
          if (!found || c.est_us < best.est_us - 1e-9) { best = c; found = true; }
        }
      }
    }
  }
  return found;
}

// Chain dot2 stage: the weights of the first steps of each wave's first item
// are loaded into LDS before the wait for the stage's X, so that the latency
// of the stage boundary streams weights.  As many whole ring groups as fit
// next to the stage's other LDS, at most the item's steps and max_steps.
void plan_wpf(Geo& g, int lds_cap, int max_steps) {
  if (g.path != 0) return;
  const int off = (int)round_up((size_t)g.lds, 1024);
  const int per_step = g.waves * g.tb * 1024;  // one 1 KB load per weight row and wave
  int q = std::min(std::min(g.steps, max_steps), (lds_cap - off) / per_step);
  q -= q % g.ring;
  if (q < g.ring) return;
  g.wpf = q;
  g.wpf_off = off;
  g.lds = off + q * per_step;
}

bool plan_kc(Geo& best, int M, int K, int N, int paired, int ntw_o, int s_o, const Cost& cost,
             int slots = kWgPerXcd, bool chain = false) {
  bool found = false;
  const int MT = std::min(4, (M + 15) / 16);  // beyond 64 rows: m-blocks of 64 (kc_geo)
  for (int ntw : {2, 3, 4, 6, 8}) {
    if (ntw_o && ntw != ntw_o) continue;
    if (ntw == 8 && MT > 2) continue;
    if (paired && ntw % 2) continue;  // a paired block holds whole (gate, up) pairs
    const int s_lo = s_o ? s_o : 1, s_hi = s_o ? s_o : 16;
    for (int s = s_lo; s <= s_hi; ++s) {
      Geo c;
      c.path = 3; c.M = M; c.K = K; c.N = N; c.ta = MT; c.tb = ntw; c.paired = paired; c.slots = slots;
      c.kc_chain = chain;
      if (!kc_geo(c, s, cost)) continue;
      if (c.S != s && !s_o) continue;
      if (!paired && !gemm_variant_exists(3, c.ta, c.tb)) continue;
      if (!found || c.est_us < best.est_us - 1e-9) { best = c; found = true; }
    }
  }
  return found;
}

}  // namespace

struct sgemm_plan_s {
  sgemm_problem prob;
  int device = 0;
  unsigned w_aux = 2;
  int sync = SYNC_AGENT;
  int grid = 8 * kWgPerXcd;
  Geo geo;                    // GEMM
  Geo cg[kChainStages];       // chain stages
  size_t ws_bytes = 0;
  size_t off_ctr = 0, off_part = 0;                 // GEMM (and chain stage 0..3 bases below)
  size_t c_ctr[kChainStages] = {0}, c_part[kChainStages] = {0};
  size_t off_lctr = 0, off_gctr = 0, off_xflag = 0, off_ready = 0, off_act = 0, off_stamps = 0;
  size_t act_layer_elems = 0, a_h1 = 0, a_h2 = 0, a_a = 0, a_x = 0;
  // Decoder layer: activations qkv = a_h1, o = a_h2, x1, a = a_a, x' = a_x; attention partials and counters.
  size_t a_x1 = 0, off_apart = 0, off_actr = 0;
  int nchunk = 0, norm_off = 0, dec_lds = 0;
  int attn_s = 1;  // decoder: attention slices (workgroups) per (sequence, head) pair
  long long spin_ticks = 0;
  int gcopies = kXcds;  // chain/decoder: copies of each global counter (see ChainArgs)
};

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels assume the device they run on: a gfx950 part with 8 XCDs of 32
// CUs each visible as one device (the grid is one workgroup per CU and the
// per-XCD partition is indexed by the hardware XCC id).  Checked once per
// device on its first run; another architecture or partition mode is
// refused with SGEMM_ERR_UNSUPPORTED instead of computing the wrong columns.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 supported, else a status

static int device_check(int device) {
  if (device < 0 || device >= kMaxDevices) return SGEMM_ERR_INVALID_ARG;
  const int st = g_device_state[device].load(std::memory_order_acquire);
  if (st == 1) return SGEMM_OK;
  if (st != 0) return st;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return SGEMM_ERR_HIP;  // not cached
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                  prop.multiProcessorCount == kXcds * kWgPerXcd;
  g_device_state[device].store(ok ? 1 : SGEMM_ERR_UNSUPPORTED, std::memory_order_release);
  return ok ? SGEMM_OK : SGEMM_ERR_UNSUPPORTED;
}

static int validate_gemm(const sgemm_problem& p) {
  if (p.M < 1 || p.K < 8 || p.N < 1) return SGEMM_ERR_INVALID_ARG;
  if (p.K % 8 != 0) return SGEMM_ERR_INVALID_ARG;
  if (p.out_dtype != SGEMM_OUT_F32 && p.out_dtype != SGEMM_OUT_BF16) return SGEMM_ERR_INVALID_ARG;
  if (p.M > kMaxM) return SGEMM_ERR_UNSUPPORTED;
  // Beyond 64 rows only the K-chunked path (64-row m-blocks) is built.
  if (p.M > 64 && (p.flags & (SGEMM_F_FORCE_DOT2 | SGEMM_F_FORCE_MFMA | SGEMM_F_MTILE_ITEMS | SGEMM_F_MSPLIT)))
    return SGEMM_ERR_UNSUPPORTED;
  if ((size_t)p.N * p.K * 2 >= kMaxOperand || (size_t)p.M * p.K * 2 >= kMaxOperand ||
      (size_t)p.M * p.N * 4 >= kMaxOperand)
    return SGEMM_ERR_UNSUPPORTED;
  return SGEMM_OK;
}

static int choose_path(const sgemm_problem& p) {
  if (p.flags & SGEMM_F_FORCE_DOT2) return 0;
  if (p.flags & SGEMM_F_FORCE_MFMA) return 1;
  return p.M < 16 ? 0 : 1;
}

static void layout_stage_ws(size_t& cursor, const Geo& g, size_t& off_ctr, size_t& off_part) {
  off_ctr = cursor;
  cursor = round_up(cursor + g.ctr_count * 4, 256);
  off_part = cursor;
  cursor = round_up(cursor + g.part_floats * 4, 256);
}

// The whole decoder layer (kind DECODER): four GEMM stages planned as the
// chain's (QKV [d -> q + 2 kv], O [q -> d], gate_up paired [d -> d_ff], down
// [d_ff -> d]) with 256 B of LDS kept for the RMSNorm factors, the attention
// stage's chunking, and the workspace layout.  Fills pl->ws_bytes.
static int plan_decoder(sgemm_plan_s* pl, const sgemm_problem& p, int tn_o, int s_o, int w_o, int k_o) {
  const unsigned refused = SGEMM_F_SYNC_FLAT | SGEMM_F_POLL_LEADER | SGEMM_F_SCHEDULER | SGEMM_F_LAUNCH_PER_STAGE |
                           SGEMM_F_W_CACHED | SGEMM_F_W_SC1 | SGEMM_F_MTILE_ITEMS | SGEMM_F_MSPLIT | SGEMM_F_KCHUNK |
                           SGEMM_F_CHECK_PLACEMENT;
  if (p.flags & refused) return SGEMM_ERR_UNSUPPORTED;
  if (p.tm) return SGEMM_ERR_INVALID_ARG;
  if (p.M < 1 || p.n_layers < 1 || p.d_model < 8 || p.d_ff < 8 || p.n_heads < 1 || p.n_kv_heads < 1 ||
      p.head_dim < 1 || p.ctx < 0)
    return SGEMM_ERR_INVALID_ARG;
  if (p.d_model % 8 || p.d_ff % 8 || p.n_heads % p.n_kv_heads) return SGEMM_ERR_INVALID_ARG;
  // Built: four query heads per key/value head, head dimension 128, up to
  // 64 attention chunks of 64 positions, M <= 64.
  if (p.n_heads / p.n_kv_heads != 4 || p.head_dim != 128) return SGEMM_ERR_UNSUPPORTED;
  if (p.M > 64 || p.n_layers > kMaxLayers || p.ctx + 1 > 64 * 64) return SGEMM_ERR_UNSUPPORTED;
  if (p.q_cols && p.q_cols != p.n_heads * p.head_dim) return SGEMM_ERR_INVALID_ARG;
  if ((p.flags & SGEMM_F_FORCE_DOT2) && p.M >= 16) return SGEMM_ERR_UNSUPPORTED;
  const size_t M = p.M, d = p.d_model, dff = p.d_ff, q = (size_t)p.n_heads * p.head_dim,
               kv = (size_t)p.n_kv_heads * p.head_dim;
  const size_t ext[] = {(q + 2 * kv) * d * 2, d * q * 2, 2 * dff * d * 2, d * dff * 2, M * (q + 2 * kv) * 2,
                        M * d * 4, M * 2 * dff * 2, M * kv * (size_t)p.ctx * 2, M * q * 2};
  for (size_t e : ext)
    if (e >= kMaxOperand) return SGEMM_ERR_UNSUPPORTED;
  const int Ks[4] = {p.d_model, (int)q, p.d_model, p.d_ff};
  const int Ns[4] = {(int)(q + 2 * kv), p.d_model, p.d_ff, p.d_model};
  Cost cost = kCostChain;
  cost.lds_reserve = 256;
  const int path = (p.flags & SGEMM_F_FORCE_DOT2) ? 0 : (p.flags & SGEMM_F_FORCE_MFMA) ? 1 : (p.M <= 2 ? 0 : 1);
  double best = -1.0;
  // dot2 stages: four columns per wave unless that cannot be planned (or tn
  // says otherwise).  Measured on the 36-layer decoder against two columns,
  // which the cost model prefers: 3.145 against 3.237 ms at M = 1 with 1024
  // positions, 3.507 against 3.565 with 4000, 3.264 against 3.333 at M = 2.
  const int tb_pref = path == 0 && !tn_o ? 4 : 0;
  for (int pass = 0; pass < 2 && best < 0.0; ++pass)
  for (int waves = 8; waves >= 4; waves -= 4) {
    if (w_o && waves != w_o) continue;
    for (int tb = 1; tb <= (path == 0 ? 4 : 2); ++tb) {
      if (path == 0 && tb != 2 && tb != 4) continue;
      if (pass == 0 && tb_pref && tb != tb_pref) continue;
      if (tn_o && tn_o != (path == 0 ? tb : 16 * tb)) continue;
      const int a = path == 0 ? p.M : (p.M + 15) / 16;
      if (!decoder_variant_exists(path, a, tb)) continue;
      Geo c[kChainStages];
      double tot = 0.0;
      bool ok = true;
      for (int s = 0; s < kChainStages && ok; ++s) {
        const int paired = s == 2;
        const int tn = path == 0 ? tb : (paired ? 0 : 16 * tb);
        if (path == 0 && k_o > 1) { ok = false; break; }
        ok = plan_geo(c[s], p.M, Ks[s], Ns[s], path, paired, tn, s_o, waves, path == 0 ? 1 : k_o, cost);
        if (ok && paired) c[s].pair_off = p.d_ff;
        tot += ok ? c[s].est_us : 0.0;
      }
      if (ok && (best < 0.0 || tot < best)) {
        best = tot;
        for (int s = 0; s < kChainStages; ++s) pl->cg[s] = c[s];
      }
    }
  }
  if (best < 0.0) return SGEMM_ERR_UNSUPPORTED;
  if (!set_chain_rr(pl->cg, kChainStages, false)) return SGEMM_ERR_INVALID_ARG;
  size_t cur = kCtl;
  for (int s = 0; s < kChainStages; ++s) {
    if (pl->cg[s].part_floats * 4 >= kMaxOperand) return SGEMM_ERR_UNSUPPORTED;
    layout_stage_ws(cur, pl->cg[s], pl->c_ctr[s], pl->c_part[s]);
  }
  const int events = 5 * p.n_layers;
  pl->off_lctr = cur;
  cur = round_up(cur + (size_t)kXcds * events * 4, 256);
  pl->off_gctr = cur;
  cur = round_up(cur + (size_t)kXcds * events * 4, 256);  // up to one copy per XCD
  pl->off_xflag = cur;
  cur = round_up(cur + (size_t)kXcds * events * 4, 256);
  pl->off_ready = cur;
  cur = round_up(cur + (size_t)kXcds * kWgPerXcd * 4, 256);
  pl->nchunk = ceil_div(p.ctx + 1, 64);
  // Attention: S workgroups (slices) per (sequence, key/value head) pair, so
  // that an XCD's 32 workgroups are busy, at most 8 and at most the chunks.
  // SGEMM_ATTN_SLICES overrides it (1..8).
  {
    const int pairs_per_xcd = ceil_div(p.n_kv_heads, kXcds) * p.M;
    int sl = 1;
    while (sl < 8 && 2 * sl * pairs_per_xcd <= kWgPerXcd && 2 * sl <= pl->nchunk) sl *= 2;
    if (!env_int("SGEMM_ATTN_SLICES", sl, &sl) || sl < 1 || sl > 8) return SGEMM_ERR_INVALID_ARG;
    pl->attn_s = sl;
  }
  const size_t apart = M * p.n_kv_heads * (size_t)pl->attn_s * 4 * (p.head_dim + 2) * 4;
  if (apart >= kMaxOperand) return SGEMM_ERR_UNSUPPORTED;
  pl->off_apart = cur;
  cur = round_up(cur + apart, 256);
  pl->off_actr = cur;
  cur = round_up(cur + M * p.n_kv_heads * 4, 256);
  pl->a_h1 = 0;                                            // qkv [M][q + 2 kv]
  pl->a_h2 = round_up(M * (q + 2 * kv), 128);             // o [M][q]
  pl->a_x1 = pl->a_h2 + round_up(M * q, 128);             // x1 [M][d]
  pl->a_a = pl->a_x1 + round_up(M * d, 128);              // a [M][d_ff]
  pl->a_x = pl->a_a + round_up(M * dff, 128);             // x' [M][d]
  pl->act_layer_elems = pl->a_x + round_up(M * d, 128);
  pl->off_act = cur;
  cur = round_up(cur + pl->act_layer_elems * 2 * p.n_layers, 256);
  pl->off_stamps = cur;
  if (p.flags & SGEMM_F_STAMPS) cur = round_up(cur + (size_t)pl->grid * events * 2 * 8, 256);
  // The attention stage: per wave queries, weights, value rows and the new
  // position's key and value rows (18.5 KB).
  int lds = 8 * (4 * 128 * 2 + 64 * 4 * 4 + 64 * 128 * 2 + 2 * 128 * 2);
  for (int s = 0; s < kChainStages; ++s) lds = std::max(lds, pl->cg[s].lds);
  pl->norm_off = (int)round_up((size_t)lds, 16);
  pl->dec_lds = pl->norm_off + 256;
  if (pl->dec_lds > kLdsMax) return SGEMM_ERR_UNSUPPORTED;
  pl->ws_bytes = cur;
  return SGEMM_OK;
}

extern "C" {

int sgemm_plan_create(const sgemm_problem* problem, int device, sgemm_plan* out,
                      size_t* workspace_bytes) {
  if (!problem || !out || !workspace_bytes) return SGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  const sgemm_problem& p = *problem;
  if ((p.flags & SGEMM_F_FORCE_DOT2) && (p.flags & SGEMM_F_FORCE_MFMA)) return SGEMM_ERR_INVALID_ARG;
  if (device < 0) return SGEMM_ERR_INVALID_ARG;
  // Overrides: the problem's fields, else the environment (0: planner's choice).
  int tn_o = p.tn, s_o = p.splitk, w_o = p.waves, k_o = p.kslices;
  if ((!tn_o && !env_int("SGEMM_TN", 0, &tn_o)) || (!s_o && !env_int("SGEMM_SPLITK", 0, &s_o)) ||
      (!w_o && !env_int("SGEMM_WAVES", 0, &w_o)) || (!k_o && !env_int("SGEMM_KSLICES", 0, &k_o)))
    return SGEMM_ERR_INVALID_ARG;
  if (tn_o < 0 || s_o < 0 || w_o < 0 || k_o < 0) return SGEMM_ERR_INVALID_ARG;
  if (w_o && w_o != 4 && w_o != 8) return SGEMM_ERR_INVALID_ARG;
  if (k_o && k_o != 1 && k_o != 2 && k_o != 4 && k_o != 8) return SGEMM_ERR_INVALID_ARG;
  if (s_o > 64) return SGEMM_ERR_UNSUPPORTED;
  double watchdog_s = 5.0;  // seconds a chain stage may wait for its producer
  if (const char* ws = std::getenv("SGEMM_WATCHDOG_S"); ws && *ws) {
    char* end = nullptr;
    watchdog_s = std::strtod(ws, &end);
    if (*end != '\0' || !(watchdog_s > 0.0 && watchdog_s <= 3600.0)) return SGEMM_ERR_INVALID_ARG;
  }

  // Chain and decoder: every XCD polls its own copy of each global counter
  // (one instruction of the XCD's releasing wave bumps all eight).  One shared
  // counter polled by all 256 workgroups (SGEMM_CHAIN_GCOPIES = 1) measured
  // 0.5-0.8% slower on the 36-layer chain at M = 1, 16 and 64.
  int gcopies = kXcds;
  if (!env_int("SGEMM_CHAIN_GCOPIES", kXcds, &gcopies) || (gcopies != 1 && gcopies != kXcds))
    return SGEMM_ERR_INVALID_ARG;

  sgemm_plan_s* pl = new (std::nothrow) sgemm_plan_s();
  if (!pl) return SGEMM_ERR_INVALID_ARG;
  pl->prob = p;
  pl->device = device;
  pl->gcopies = gcopies;
  pl->w_aux = (p.flags & SGEMM_F_W_CACHED) ? 0u : ((p.flags & SGEMM_F_W_SC1) ? 18u : 2u);
  pl->sync = (p.flags & SGEMM_F_SYNC_AGENT) ? SYNC_AGENT : SYNC_XCD;

  size_t cur = kCtl;
  if (p.kind == SGEMM_KIND_GEMM) {
    if (p.flags & SGEMM_F_SCHEDULER) { delete pl; return SGEMM_ERR_UNSUPPORTED; }  // a chain runtime
    int rc = validate_gemm(p);
    if (rc != SGEMM_OK) { delete pl; return rc; }
    const bool msplit = (p.flags & SGEMM_F_MSPLIT) != 0;
    const bool mti = (p.flags & SGEMM_F_MTILE_ITEMS) != 0 || msplit;
    const bool kc = (p.flags & SGEMM_F_KCHUNK) != 0;
    // Beyond 64 rows: the large-tile path unless the K-chunked one is asked
    // for (SGEMM_LT=0 takes the K-chunked path there too).
    // SGEMM_LT_MIN_M: the fewest rows that take the large-tile path (65 by
    // default; from 16 it replaces the MFMA paths too).
    int lt_env = 1, lt_min = 65;
    if (!env_int("SGEMM_LT", 1, &lt_env) || !env_int("SGEMM_LT_MIN_M", 65, &lt_min)) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    const bool lt = p.M >= std::max(lt_min, 16) && !kc && lt_env && !(p.flags & (SGEMM_F_FORCE_DOT2 | SGEMM_F_FORCE_MFMA | SGEMM_F_MTILE_ITEMS | SGEMM_F_MSPLIT));
    const bool kcm = kc || (p.M > 64 && !lt);
    // Rows per m-tile item (the window of the M-major traversal): 16 unless given.
    const int mti_rows = !mti ? 0 : (p.tm ? p.tm : 16);
    if (mti && mti_rows != 16 && mti_rows != 32 && mti_rows != 64) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if (!mti && p.tm && !(lt && (p.tm == 64 || p.tm == 128 || p.tm == 256))) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if ((mti || kc) && (p.flags & SGEMM_F_FORCE_DOT2)) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if (mti && kc) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    const int path = mti ? 1 : choose_path(p);
    if ((path == 0 || mti || kcm || lt) && k_o > 1) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    // The K-chunked and large-tile kernels are built with nontemporal weight loads only.
    const bool nt_w = pl->w_aux == 2u;
    if (lt) {
      // tn gives the workgroup tile's columns (96, 192 or 384), tm its rows
      // (64, 128 or 256), waves 4 or 8.
      // Weights nt or with the default policy (SGEMM_F_W_CACHED), not sc1.
      if ((w_o && w_o != 4 && w_o != 8) || (p.flags & SGEMM_F_W_SC1)) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
      if (!plan_lt(pl->geo, p.M, p.K, p.N, p.tm, tn_o, w_o, s_o)) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
      // Several m-blocks read each weight line (R >= 2 in Eq.(1) of the
      // Fleet reading note, section 3f): the default cache policy keeps the
      // lines in L2 for the later readers (measured: 256 x 4096 x 24576 67.1
      // against 75.5 us, HBM fetch 1.09 against 1.25 x the weights;
      // 256 x 12288 x 4096 52.3 against 60.4 us); one reader keeps nt.
      if (pl->geo.mb > 1) pl->w_aux = 0u;
    } else if (kcm) {
      // tn (a multiple of 16) gives the tiles per item.
      if (tn_o % 16 || w_o == 4 || !nt_w) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
      if (!plan_kc(pl->geo, p.M, p.K, p.N, 0, tn_o / 16, s_o, kCostGemm)) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    } else if (!plan_geo(pl->geo, p.M, p.K, p.N, path, 0, tn_o, s_o, w_o, k_o, kCostGemm, 0, mti_rows)) {
      delete pl;
      return SGEMM_ERR_UNSUPPORTED;
    } else if (path == 1 && !mti && nt_w && !tn_o && !s_o && !w_o && !k_o && p.M > 48 &&
               (p.N >= 12288 || p.K >= 12288)) {
      // Four full m-tiles on the widest shapes: the large-tile path with a
      // 64 x 96 tile and four waves (measured, cold HBM: 64 x 4096 x 24576
      // 46.0 against 49.8 us on the K-chunked path, 64 x 12288 x 4096 32.7
      // against 35.8 us on the split MFMA path; on the 4096-column shapes
      // and at M = 32 it was slower).
      Geo ltg;
      if (plan_lt(ltg, p.M, p.K, p.N, 64, 96, 4, 0)) pl->geo = ltg;
    } else if (path == 1 && !mti && nt_w && !tn_o && !s_o && !w_o && !k_o && (p.K >= 6144 || p.M > 48)) {
      // Long K, or four full m-tiles, with a wide output: the K-chunked path
      // takes one item of six tiles over all of K per workgroup and needs no
      // split-K, where the windowed MFMA path has to split K four to seven
      // ways (measured, back-to-back launches: 16 x 7168 x 18432 45.0 against
      // 47.6 us, 64 x 4096 x 24576 49.5 against 54.0 us; at M = 32 and 48 and
      // on the narrower outputs it measured no faster).
      Geo kcg;
      if (plan_kc(kcg, p.M, p.K, p.N, 0, 6, 1, kCostGemm) && kcg.items <= kWgPerXcd &&
          kcg.items * 4 >= kWgPerXcd * 3 && pl->geo.S > 2)
        pl->geo = kcg;
    } else if (path == 1 && !mti && nt_w && !tn_o && !s_o && !w_o && !k_o && p.M > 16 && p.M <= 48 &&
               p.K > 3072 && p.K <= 4096 && p.N <= 4096 && pl->geo.S < 4) {
      // Two or three m-tiles on a 4096-deep output of at most 4096 columns:
      // four K splits instead of the cost model's one or two, so the X window
      // each workgroup fills before its first step drops from 128-147 KB to
      // 64 KB for 0.5-1 MB of partials (measured, cold HBM, best of 60
      // launches: 17 x 4096 x 4096 15.96 -> 14.24 us, 24 x 4096 x 4096
      // 14.88 -> 14.32, 32 x 4096 x 4096 15.56 -> 14.60, 32 x 4096 x 2048
      // 14.76 -> 12.88, 36 x 4096 x 2048 15.68 -> 13.40; at K = 3072 and on
      // 6144-wide outputs within -9..+10%, so left alone).
      Geo g4;
      if (plan_geo(g4, p.M, p.K, p.N, path, 0, 0, 4, 0, 0, kCostGemm)) pl->geo = g4;
    } else if (path == 0 && nt_w && !tn_o && !s_o && !w_o && !k_o && p.M >= 10 && p.M < 16 &&
               p.K >= 6144 && p.K <= 8192 && p.N >= 3072 && p.N <= 4096 && pl->geo.S > 2) {
      // dot2 at M = 10-15 where the X window over all of K does not fit:
      // two K splits instead of the cost model's four (measured, cold HBM,
      // best of 60 launches: 12 x 7168 x 4096 25.32 -> 22.40 us, 15 x 7168 x
      // 4096 27.88 -> 24.84, 12 x 7168 x 3072 22.04 -> 19.44, 15 x 8192 x
      // 4096 28.96 -> 27.48, 15 x 6144 x 4096 27.88 -> 25.08; on 1536-wide
      // outputs and at M = 8 four splits measured as fast or faster).
      Geo g2;
      if (plan_geo(g2, p.M, p.K, p.N, path, 0, 0, 2, 0, 0, kCostGemm)) pl->geo = g2;
    }
    if ((pl->geo.path == 3 || pl->geo.path == 5 || pl->geo.path == 6) && pl->geo.mb > 1) {
      // m-blocks round-robin over the XCD's workgroups (shared weights in
      // L2); SGEMM_KC_RR=0 gives each workgroup a contiguous range instead.
      int rr = 1;
      if (!env_int("SGEMM_KC_RR", 1, &rr)) { delete pl; return SGEMM_ERR_INVALID_ARG; }
      pl->geo.rr = rr ? 1 : 0;
    }
    pl->geo.nfast = msplit ? 1 : 0;
    if ((pl->geo.path == 0 || (pl->geo.path == 1 && pl->geo.mtiles == 1)) && pl->geo.S == 1) {
      // Items round-robin over the XCD's streams (measured 0-3% faster than
      // contiguous ranges on the dot2 decode shapes, 2-5% on M = 16 MFMA
      // ones with several items per workgroup; bitwise the same results);
      // SGEMM_DOT2_RR=0 / SGEMM_MFMA_RR=0 keep the contiguous ranges.
      int rr = 1;
      if (!env_int(pl->geo.path == 0 ? "SGEMM_DOT2_RR" : "SGEMM_MFMA_RR", 1, &rr)) { delete pl; return SGEMM_ERR_INVALID_ARG; }
      pl->geo.rr = rr ? 1 : 0;
    }
    if (pl->geo.part_floats * 4 >= kMaxOperand) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    layout_stage_ws(cur, pl->geo, pl->off_ctr, pl->off_part);
  } else if (p.kind == SGEMM_KIND_LAYERCHAIN) {
    if (p.tm || (p.flags & (SGEMM_F_W_CACHED | SGEMM_F_W_SC1 | SGEMM_F_MTILE_ITEMS | SGEMM_F_CHECK_PLACEMENT |
                            SGEMM_F_MSPLIT))) {
      delete pl;
      return SGEMM_ERR_UNSUPPORTED;
    }
    const bool kcf = (p.flags & SGEMM_F_KCHUNK) != 0;
    if (kcf && ((p.flags & (SGEMM_F_FORCE_DOT2 | SGEMM_F_FORCE_MFMA)) || k_o > 1 || (w_o && w_o != 8)))
      { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    const bool sched = (p.flags & SGEMM_F_SCHEDULER) != 0;
    if (sched && (p.flags & (SGEMM_F_SYNC_FLAT | SGEMM_F_POLL_LEADER))) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    const int slots = sched ? kWgPerXcd - 1 : kWgPerXcd;  // the scheduler workgroup takes no items
    if (p.M < 1 || p.n_layers < 1 || p.d_model < 8 || p.q_cols < 8 || p.d_ff < 8)
      { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if (p.d_model % 8 || p.q_cols % 8 || p.d_ff % 8) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if (p.M > 64 || p.n_layers > kMaxLayers) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    // Every operand a stage addresses through a buffer descriptor must stay
    // below the 31-bit extent: weights, X and Y of each stage, the fp32 copy
    // of the last output.
    {
      const size_t M_ = (size_t)p.M, d_ = (size_t)p.d_model, q_ = (size_t)p.q_cols, f_ = (size_t)p.d_ff;
      const size_t ext[] = {q_ * d_ * 2, d_ * q_ * 2, 2 * f_ * d_ * 2, d_ * f_ * 2,
                            M_ * d_ * 4, M_ * q_ * 2, M_ * 2 * f_ * 2};
      for (size_t e : ext)
        if (e >= kMaxOperand) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    }
    // Stages: Q [d -> q], O [q -> d], gate_up paired [d -> dff], down [dff -> d].
    // One block size and one n-tile width for the unpaired stages per launch.
    const int Ks[4] = {p.d_model, p.q_cols, p.d_model, p.d_ff};
    const int Ns[4] = {p.q_cols, p.d_model, p.d_ff, p.d_model};
    // Per-stage overrides for experiments: SGEMM_CHAIN_S / _KSL / _WPI =
    // four comma-separated values (Q, O, gate_up, down), 0 = planner's choice.
    int s_st[4] = {s_o, s_o, s_o, s_o}, k_st[4] = {k_o, k_o, k_o, k_o}, w_st[4] = {0, 0, 0, 0};
    for (int which = 0; which < 3; ++which) {
      const char* e = std::getenv(which == 0 ? "SGEMM_CHAIN_S" : which == 1 ? "SGEMM_CHAIN_KSL" : "SGEMM_CHAIN_WPI");
      if (!e || !*e) continue;
      int v[4] = {0, 0, 0, 0};
      if (std::sscanf(e, "%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3]) != 4) { delete pl; return SGEMM_ERR_INVALID_ARG; }
      for (int i = 0; i < 4; ++i)
        if (v[i]) (which == 0 ? s_st : which == 1 ? k_st : w_st)[i] = v[i];
    }
    // SGEMM_CHAIN_COST = "alpha,x_gbps,split_us,fin_us_kb,ksl_us" replaces the chain's
    // cost constants (for calibration runs).
    Cost cost = kCostChain;
    if (const char* ce = std::getenv("SGEMM_CHAIN_COST"); ce && *ce) {
      double x_gbps = 0.0;
      if (std::sscanf(ce, "%lf,%lf,%lf,%lf,%lf", &cost.alpha, &x_gbps, &cost.split_us, &cost.fin_us_kb,
                      &cost.ksl_us) != 5 ||
          !(cost.alpha >= 1.0 && cost.alpha <= 8.0) || !(x_gbps > 0.0) || cost.split_us < 0.0 ||
          cost.fin_us_kb < 0.0 || cost.ksl_us < 0.0) {
        delete pl;
        return SGEMM_ERR_INVALID_ARG;
      }
      cost.x_bw = x_gbps * 1e9;
    }
    // dot2 stages (G weight rows per wave, the gate_up stage holding G/2
    // gate/up pairs) at M <= 2, MFMA stages above: in the 36-layer chain the
    // dot2 stages measured 4% faster at M = 1, even at M = 2 and 2-45% slower
    // from M = 3 to 15.  SGEMM_F_FORCE_DOT2 (M < 16) and SGEMM_F_FORCE_MFMA
    // choose the path.
    if ((p.flags & SGEMM_F_FORCE_DOT2) && p.M >= 16) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    const int path = (p.flags & SGEMM_F_FORCE_DOT2) ? 0 : (p.flags & SGEMM_F_FORCE_MFMA) ? 1 : (p.M <= 2 ? 0 : 1);
    double best = -1.0;
    // SGEMM_F_KCHUNK: every stage on the K-chunked MFMA path, NTW_u tiles per
    // item in the Q, O and down stages and NTW_p in gate_up (kernel code
    // 10 NTW_u + NTW_p); a tile-width override fixes NTW_u = tn / 16.
    const int MTk = (p.M + 15) / 16;
    for (int nu = 2; kcf && nu <= 6; nu += 2) {
      for (int np = 4; np <= 6; np += 2) {
        if (tn_o && tn_o != 16 * nu) continue;
        if (!chain_variant_exists(3, MTk, 10 * nu + np)) continue;
        Geo c[kChainStages];
        double tot = 0.0;
        bool ok = true;
        for (int s = 0; s < kChainStages && ok; ++s) {
          const int paired = s == 2;
          ok = plan_kc(c[s], p.M, Ks[s], Ns[s], paired, paired ? np : nu, s_st[s], cost, slots, true);
          if (ok && paired) c[s].pair_off = p.d_ff;
          tot += ok ? c[s].est_us : 0.0;
        }
        if (ok && (best < 0.0 || tot < best)) {
          best = tot;
          for (int s = 0; s < kChainStages; ++s) pl->cg[s] = c[s];
        }
      }
    }
    for (int waves = 8; !kcf && waves >= 4; waves -= 4) {
      if (w_o && waves != w_o) continue;
      for (int nt = 1; nt <= (path == 0 ? 4 : 2); ++nt) {
        // dot2: G = 2 or 4 rows per wave in every stage; MFMA: NT = 1 or 2.
        const int tb = nt;
        if (path == 0 && tb != 2 && tb != 4) continue;
        if (tn_o && tn_o != (path == 0 ? tb : 16 * tb)) continue;
        const int a = path == 0 ? p.M : (p.M + 15) / 16;
        Geo c[kChainStages];
        double tot = 0.0;
        bool ok = chain_variant_exists(path, a, tb);
        for (int s = 0; s < kChainStages && ok; ++s) {
          const int paired = s == 2;
          const int tn = path == 0 ? tb : (paired ? 0 : 16 * tb);
          if (path == 0 && k_st[s] > 1) { ok = false; break; }  // no K slices on the dot2 path
          ok = plan_geo(c[s], p.M, Ks[s], Ns[s], path, paired, tn, s_st[s], waves, path == 0 ? 1 : k_st[s], cost,
                        w_st[s], false, slots);
          if (ok && paired) c[s].pair_off = p.d_ff;
          tot += ok ? c[s].est_us : 0.0;
        }
        if (ok && (best < 0.0 || tot < best)) {
          best = tot;
          for (int s = 0; s < kChainStages; ++s) pl->cg[s] = c[s];
        }
      }
    }
    if (best < 0.0) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    for (int s = 0; s < kChainStages; ++s)
      if (pl->cg[s].part_floats * 4 >= kMaxOperand) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    // Ablation: SGEMM_CHAIN_WPF = n loads up to n weight steps into LDS
    // ahead of each dot2 stage's wait (default 0, none).  The extra traffic at
    // the stage boundary slows the counters' round trips and the X loads by
    // more than it saves: the 36-layer chain at M = 1 and 2 measured 0-6%
    // slower with 4 or 8 steps.
    int wpf_max = 0;
    if (!env_int("SGEMM_CHAIN_WPF", 0, &wpf_max) || wpf_max < 0) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    for (int s = 0; s < kChainStages; ++s) plan_wpf(pl->cg[s], kLdsMax, wpf_max);
    if (!set_chain_rr(pl->cg, kChainStages, (p.flags & SGEMM_F_SCHEDULER) != 0)) {
      delete pl;
      return SGEMM_ERR_INVALID_ARG;
    }
    // Re-layout with the final geometries.
    cur = kCtl;
    for (int s = 0; s < kChainStages; ++s) layout_stage_ws(cur, pl->cg[s], pl->c_ctr[s], pl->c_part[s]);
    const int events = kChainStages * p.n_layers;
    pl->off_lctr = cur;
    cur = round_up(cur + (size_t)kXcds * events * 4, 256);
    pl->off_gctr = cur;
    cur = round_up(cur + (size_t)kXcds * events * 4, 256);  // up to one copy per XCD
    pl->off_xflag = cur;
    cur = round_up(cur + (size_t)kXcds * events * 4, 256);
    pl->off_ready = cur;
    cur = round_up(cur + (size_t)kXcds * kWgPerXcd * 4, 256);
    const size_t M = p.M;
    pl->a_h1 = 0;
    pl->a_h2 = round_up(M * p.q_cols, 128);
    pl->a_a = pl->a_h2 + round_up(M * p.d_model, 128);
    pl->a_x = pl->a_a + round_up(M * p.d_ff, 128);
    pl->act_layer_elems = pl->a_x + round_up(M * p.d_model, 128);
    pl->off_act = cur;
    cur = round_up(cur + pl->act_layer_elems * 2 * p.n_layers, 256);
    pl->off_stamps = cur;
    if (p.flags & SGEMM_F_STAMPS) cur = round_up(cur + (size_t)pl->grid * events * 2 * 8, 256);
    pl->spin_ticks = (p.flags & SGEMM_F_WATCHDOG_TEST) ? 0 : (long long)(watchdog_s * 1.0e8);
  } else if (p.kind == SGEMM_KIND_DECODER) {
    const int rc = plan_decoder(pl, p, tn_o, s_o, w_o, k_o);
    if (rc != SGEMM_OK) { delete pl; return rc; }
    cur = pl->ws_bytes;
    pl->spin_ticks = (p.flags & SGEMM_F_WATCHDOG_TEST) ? 0 : (long long)(watchdog_s * 1.0e8);
  } else {
    delete pl;
    return SGEMM_ERR_INVALID_ARG;
  }
  pl->ws_bytes = std::max(cur, (size_t)4096);
  *workspace_bytes = pl->ws_bytes;
  *out = pl;
  return SGEMM_OK;
}

int sgemm_plan_destroy(sgemm_plan plan) {
  delete plan;
  return SGEMM_OK;
}

int sgemm_workspace_init(sgemm_plan plan, void* workspace, void* stream) {
  if (!plan || !workspace || !aligned16(workspace)) return SGEMM_ERR_INVALID_ARG;
  if (hipSetDevice(plan->device) != hipSuccess) return SGEMM_ERR_HIP;
  return launch_fill_zero(workspace, plan->ws_bytes, (hipStream_t)stream) == hipSuccess ? SGEMM_OK
                                                                                        : SGEMM_ERR_HIP;
}

static StageDesc stage_desc(const Geo& g, unsigned w_aux, int sync) {
  StageDesc d;
  std::memset(&d, 0, sizeof d);
  d.M = g.M; d.K = g.K; d.N = g.N;
  d.Nx = g.Nx; d.TN = g.TN; d.wpi = g.wpi; d.ng = g.ng; d.CB = g.CB; d.NB = g.NB; d.S = g.S;
  d.KS = g.KS; d.ksl = g.ksl; d.kss = g.kss;
  d.steps = g.steps; d.items = g.items; d.win = g.win; d.xrow = g.xrow;
  d.red_off = g.red_off; d.stash_off = g.stash_off; d.stash_cap = g.stash_cap;
  d.pair_off = g.pair_off;
  d.mtiles = g.mtiles;
  d.interleave = g.mtiles > 1 ? 1 : 0;
  d.rr = g.rr;
  d.nfast = g.nfast;
  d.xbuf = g.xbuf;
  d.mb = g.mb;
  d.nctr = (int)g.ctr_count;
  d.wpf = g.wpf;
  d.wpf_off = g.wpf_off;
  d.w_aux = w_aux;
  d.sync = sync;
  return d;
}

// One single-GEMM launch with the workspace's control block at ws, its split-K
// counters at ws + off_ctr and its partials at ws + off_part (arguments
// already checked).
static int launch_plan_gemm(sgemm_plan plan, const void* X, const void* W, void* Y, char* ws, size_t off_ctr,
                            size_t off_part, void* stream) {
  const sgemm_problem& p = plan->prob;
  const Geo& g = plan->geo;
  StageDesc d = stage_desc(g, plan->w_aux, plan->sync);
  d.X = (const uint16_t*)X;
  d.W = (const uint16_t*)W;
  d.Y = Y;
  d.Y2 = nullptr;
  d.ldx = p.K;
  d.ldy = p.N;
  d.mode = p.out_dtype == SGEMM_OUT_F32 ? OUT_F32 : OUT_BF16;
  d.check = (p.flags & SGEMM_F_CHECK_PLACEMENT) ? 1 : 0;
  d.part = (float*)(ws + off_part);
  d.part_bytes = (unsigned)(g.part_floats * 4);
  d.ctr = (unsigned*)(ws + off_ctr);
  d.x_bytes = (unsigned)((size_t)p.M * p.K * 2);
  d.w_bytes = (unsigned)((size_t)p.N * p.K * 2);
  d.y_bytes = (unsigned)((size_t)p.M * p.N * (p.out_dtype == SGEMM_OUT_F32 ? 4 : 2));
  d.y2_bytes = 0;
  if (const int dc = device_check(plan->device); dc != SGEMM_OK) return dc;
  if (hipSetDevice(plan->device) != hipSuccess) return SGEMM_ERR_HIP;
  hipError_t e = launch_gemm(d, g.mtiles > 1 ? 2 : g.path, g.ta, g.tb, plan->grid, g.waves * 64, g.lds, (unsigned*)ws,
                             (hipStream_t)stream);
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

int sgemm_run(sgemm_plan plan, const void* X, const void* W, void* Y, void* workspace, void* stream) {
  if (!plan || !X || !W || !Y || !workspace) return SGEMM_ERR_INVALID_ARG;
  if (plan->prob.kind != SGEMM_KIND_GEMM) return SGEMM_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || !aligned16(workspace))
    return SGEMM_ERR_INVALID_ARG;
  return launch_plan_gemm(plan, X, W, Y, (char*)workspace, plan->off_ctr, plan->off_part, stream);
}

// ------------------------------------------------------------------------
// The single GEMM over a library-owned device array instead of a caller's
// workspace, for callers that cannot allocate.  Layout of the array, fixed
// for every plan: the control block, then a counter region, then the
// partials.  Every run leaves its split-K counters at zero (each is reset by
// its tile's last arriver) and the array is zero when the code object is
// loaded, so the counter region is all zeros before every run whatever plan
// ran before; the partials need no initial value.  Each GPU holds its own
// copy, found once per device with hipGetSymbolAddress.
namespace {
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;  // per device, held until the process ends
constexpr size_t kStaticCtrBytes = (size_t)1 << 20;       // split-K counters: 262144
constexpr size_t kStaticPartBytes = kStaticScratchBytes - kCtl - kStaticCtrBytes;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// The device address of this device's copy of `scratch` (looked up on the
// first call for the device, with the device current).
static int scratch_of(int device, char** out) {
  if (device < 0 || device >= kMaxDevices) return SGEMM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SGEMM_ERR_HIP;
    if (hipSetDevice(device) != hipSuccess) return SGEMM_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (hipSetDevice(cur) != hipSuccess || e != hipSuccess || !ptr) return SGEMM_ERR_HIP;
    g_scratch_ptr[device] = ptr;
  }
  *out = (char*)g_scratch_ptr[device];
  return SGEMM_OK;
}

int sgemm_run_noalloc(sgemm_plan plan, const void* X, const void* W, void* Y, void* stream) {
  if (!plan || !X || !W || !Y) return SGEMM_ERR_INVALID_ARG;
  if (plan->prob.kind != SGEMM_KIND_GEMM) return SGEMM_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return SGEMM_ERR_INVALID_ARG;
  // No status word is read back for the shared array.
  if (plan->prob.flags & SGEMM_F_CHECK_PLACEMENT) return SGEMM_ERR_UNSUPPORTED;
  if (plan->geo.ctr_count * 4 > kStaticCtrBytes || plan->geo.part_floats * 4 > kStaticPartBytes)
    return SGEMM_ERR_WORKSPACE;
  if (const int dc = device_check(plan->device); dc != SGEMM_OK) return dc;
  char* ws = nullptr;
  if (const int rc = scratch_of(plan->device, &ws); rc != SGEMM_OK) return rc;
  return launch_plan_gemm(plan, X, W, Y, ws, kCtl, kCtl + kStaticCtrBytes, stream);
}

int layerchain_run(sgemm_plan plan, const void* X0, const void* const* Wq, const void* const* Wo,
                   const void* const* Wgu, const void* const* Wdown, float* Y_f32, void* Y_bf16,
                   void* workspace, void* stream) {
  if (!plan || !X0 || !Wq || !Wo || !Wgu || !Wdown || !Y_f32 || !workspace)
    return SGEMM_ERR_INVALID_ARG;
  const sgemm_problem& p = plan->prob;
  if (p.kind != SGEMM_KIND_LAYERCHAIN) return SGEMM_ERR_INVALID_ARG;
  if (!aligned16(X0) || !aligned16(Y_f32) || !aligned16(workspace) || (Y_bf16 && !aligned16(Y_bf16)))
    return SGEMM_ERR_INVALID_ARG;
  ChainArgs a;
  std::memset(&a, 0, sizeof a);
  for (int l = 0; l < p.n_layers; ++l) {
    if (!Wq[l] || !Wo[l] || !Wgu[l] || !Wdown[l]) return SGEMM_ERR_INVALID_ARG;
    if (!aligned16(Wq[l]) || !aligned16(Wo[l]) || !aligned16(Wgu[l]) || !aligned16(Wdown[l]))
      return SGEMM_ERR_INVALID_ARG;
    a.wq[l] = (const uint16_t*)Wq[l];
    a.wo[l] = (const uint16_t*)Wo[l];
    a.wgu[l] = (const uint16_t*)Wgu[l];
    a.wdown[l] = (const uint16_t*)Wdown[l];
  }
  char* ws = (char*)workspace;
  const int Ks[4] = {p.d_model, p.q_cols, p.d_model, p.d_ff};
  const int Ns[4] = {p.q_cols, p.d_model, p.d_ff, p.d_model};
  const int Wrows[4] = {p.q_cols, p.d_model, 2 * p.d_ff, p.d_model};
  for (int s = 0; s < kChainStages; ++s) {
    StageDesc d = stage_desc(plan->cg[s], plan->w_aux, plan->sync);
    d.part = (float*)(ws + plan->c_part[s]);
    d.part_bytes = (unsigned)(plan->cg[s].part_floats * 4);
    d.ctr = (unsigned*)(ws + plan->c_ctr[s]);
    d.ldx = Ks[s];
    d.ldy = Ns[s];
    d.x_bytes = (unsigned)((size_t)p.M * Ks[s] * 2);
    d.w_bytes = (unsigned)((size_t)Wrows[s] * Ks[s] * 2);
    d.y_bytes = (unsigned)((size_t)p.M * Ns[s] * 2);
    d.mode = s == 2 ? OUT_SILU_BF16 : OUT_BF16;
    d.y2_bytes = s == 3 ? (unsigned)((size_t)p.M * p.d_model * 4) : 0u;
    a.st[s] = d;
  }
  a.x0 = (const uint16_t*)X0;
  a.act = (uint16_t*)(ws + plan->off_act);
  a.y_f32 = Y_f32;
  a.y_bf16 = (uint16_t*)Y_bf16;
  a.status = (unsigned*)ws;
  a.done = (unsigned*)(ws + 64);
  a.claim = (unsigned*)(ws + 128);
  a.lctr = (unsigned*)(ws + plan->off_lctr);
  a.gctr = (unsigned*)(ws + plan->off_gctr);
  a.xflag = (unsigned*)(ws + plan->off_xflag);
  a.ready = (unsigned*)(ws + plan->off_ready);
  a.stamps = (p.flags & SGEMM_F_STAMPS) ? (unsigned long long*)(ws + plan->off_stamps) : nullptr;
  a.n_layers = p.n_layers; a.M = p.M; a.d = p.d_model; a.q = p.q_cols; a.dff = p.d_ff;
  a.spl = kChainStages;
  a.act_layer_elems = plan->act_layer_elems;
  a.off_h1 = plan->a_h1; a.off_h2 = plan->a_h2; a.off_a = plan->a_a; a.off_x = plan->a_x;
  a.flat_sync = (p.flags & SGEMM_F_SYNC_FLAT) ? 1 : 0;
  a.poll_leader = (p.flags & SGEMM_F_POLL_LEADER) ? 1 : 0;
  a.sched = (p.flags & SGEMM_F_SCHEDULER) ? 1 : 0;
  a.spin_ticks = plan->spin_ticks;
  a.gcopies = plan->gcopies;
  a.path = plan->cg[0].path;
  a.mt = plan->cg[0].ta;
  a.nt_q = plan->cg[0].tb; a.nt_o = plan->cg[1].tb; a.nt_d = plan->cg[3].tb;
  if (a.path == 3) a.nt_q = 10 * plan->cg[0].tb + plan->cg[2].tb;  // K-chunked kernel code
  int lds = 0;
  for (int s = 0; s < kChainStages; ++s) lds = std::max(lds, plan->cg[s].lds);
  if (const int dc = device_check(plan->device); dc != SGEMM_OK) return dc;
  if (hipSetDevice(plan->device) != hipSuccess) return SGEMM_ERR_HIP;
  // One launch runs every event; the per-stage ablation launches once per event.
  const int events = 4 * p.n_layers;
  const int per_launch = (p.flags & SGEMM_F_LAUNCH_PER_STAGE) ? 1 : events;
  hipError_t e = hipSuccess;
  for (int e0 = 0; e0 < events && e == hipSuccess; e0 += per_launch) {
    a.e_begin = e0;
    a.e_end = e0 + per_launch;
    e = launch_chain(a, plan->grid, plan->cg[0].waves * 64, lds, (hipStream_t)stream);
  }
  if (e == hipSuccess && Y_bf16) {
    const size_t off = plan->off_act + ((size_t)(p.n_layers - 1) * plan->act_layer_elems + plan->a_x) * 2;
    e = hipMemcpyAsync(Y_bf16, ws + off, (size_t)p.M * p.d_model * 2, hipMemcpyDeviceToDevice,
                       (hipStream_t)stream);
  }
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

int decoder_run(sgemm_plan plan, const void* X0, const void* w_norm, const void* const* Wqkv, const void* const* Wo,
                const void* const* Wgu, const void* const* Wdown, const void* K_cache, const void* V_cache,
                float* Y_f32, void* Y_bf16, void* workspace, void* stream) {
  if (!plan || !X0 || !w_norm || !Wqkv || !Wo || !Wgu || !Wdown || !Y_f32 || !workspace) return SGEMM_ERR_INVALID_ARG;
  const sgemm_problem& p = plan->prob;
  if (p.kind != SGEMM_KIND_DECODER) return SGEMM_ERR_INVALID_ARG;
  if (p.ctx > 0 && (!K_cache || !V_cache)) return SGEMM_ERR_INVALID_ARG;
  if (!aligned16(X0) || !aligned16(w_norm) || !aligned16(Y_f32) || !aligned16(workspace) ||
      (Y_bf16 && !aligned16(Y_bf16)) || (K_cache && !aligned16(K_cache)) || (V_cache && !aligned16(V_cache)))
    return SGEMM_ERR_INVALID_ARG;
  ChainArgs a;
  std::memset(&a, 0, sizeof a);
  for (int l = 0; l < p.n_layers; ++l) {
    if (!Wqkv[l] || !Wo[l] || !Wgu[l] || !Wdown[l]) return SGEMM_ERR_INVALID_ARG;
    if (!aligned16(Wqkv[l]) || !aligned16(Wo[l]) || !aligned16(Wgu[l]) || !aligned16(Wdown[l]))
      return SGEMM_ERR_INVALID_ARG;
    a.wq[l] = (const uint16_t*)Wqkv[l];
    a.wo[l] = (const uint16_t*)Wo[l];
    a.wgu[l] = (const uint16_t*)Wgu[l];
    a.wdown[l] = (const uint16_t*)Wdown[l];
  }
  char* ws = (char*)workspace;
  const int q = p.n_heads * p.head_dim, kv = p.n_kv_heads * p.head_dim;
  const int Ks[4] = {p.d_model, q, p.d_model, p.d_ff};
  const int Ns[4] = {q + 2 * kv, p.d_model, p.d_ff, p.d_model};
  const int Wrows[4] = {q + 2 * kv, p.d_model, 2 * p.d_ff, p.d_model};
  for (int s = 0; s < kChainStages; ++s) {
    StageDesc d = stage_desc(plan->cg[s], plan->w_aux, plan->sync);
    d.part = (float*)(ws + plan->c_part[s]);
    d.part_bytes = (unsigned)(plan->cg[s].part_floats * 4);
    d.ctr = (unsigned*)(ws + plan->c_ctr[s]);
    d.ldx = Ks[s];
    d.ldy = Ns[s];
    d.x_bytes = (unsigned)((size_t)p.M * Ks[s] * 2);
    d.w_bytes = (unsigned)((size_t)Wrows[s] * Ks[s] * 2);
    d.y_bytes = (unsigned)((size_t)p.M * Ns[s] * 2);
    d.r_bytes = (unsigned)((size_t)p.M * Ns[s] * 2);
    d.mode = s == 2 ? OUT_SILU_BF16 : OUT_BF16;
    d.y2_bytes = s == 3 ? (unsigned)((size_t)p.M * p.d_model * 4) : 0u;
    a.st[s] = d;
  }
  a.x0 = (const uint16_t*)X0;
  a.act = (uint16_t*)(ws + plan->off_act);
  a.y_f32 = Y_f32;
  a.y_bf16 = (uint16_t*)Y_bf16;
  a.status = (unsigned*)ws;
  a.done = (unsigned*)(ws + 64);
  a.claim = (unsigned*)(ws + 128);
  a.lctr = (unsigned*)(ws + plan->off_lctr);
  a.gctr = (unsigned*)(ws + plan->off_gctr);
  a.xflag = (unsigned*)(ws + plan->off_xflag);
  a.ready = (unsigned*)(ws + plan->off_ready);
  a.stamps = (p.flags & SGEMM_F_STAMPS) ? (unsigned long long*)(ws + plan->off_stamps) : nullptr;
  a.n_layers = p.n_layers; a.M = p.M; a.d = p.d_model; a.q = q; a.dff = p.d_ff;
  a.spl = 5;
  a.act_layer_elems = plan->act_layer_elems;
  a.off_qkv = plan->a_h1; a.off_o = plan->a_h2; a.off_x1 = plan->a_x1; a.off_a = plan->a_a; a.off_x = plan->a_x;
  a.wnorm = (const uint16_t*)w_norm;
  a.kc = (const uint16_t*)K_cache;
  a.vc = (const uint16_t*)V_cache;
  a.apart = (float*)(ws + plan->off_apart);
  a.actr = (unsigned*)(ws + plan->off_actr);
  a.Hq = p.n_heads; a.Hkv = p.n_kv_heads; a.hd = p.head_dim; a.T = p.ctx; a.pc = 64; a.nchunk = plan->nchunk;
  a.attn_s = plan->attn_s;
  a.eps = 1e-6f;
  a.norm_off = plan->norm_off;
  a.spin_ticks = plan->spin_ticks;
  a.gcopies = plan->gcopies;
  a.path = plan->cg[0].path;
  a.mt = plan->cg[0].ta;
  a.nt_q = plan->cg[0].tb; a.nt_o = plan->cg[1].tb; a.nt_d = plan->cg[3].tb;
  a.e_begin = 0;
  a.e_end = 5 * p.n_layers;
  if (const int dc = device_check(plan->device); dc != SGEMM_OK) return dc;
  if (hipSetDevice(plan->device) != hipSuccess) return SGEMM_ERR_HIP;
  hipError_t e = launch_decoder(a, plan->grid, plan->cg[0].waves * 64, plan->dec_lds, (hipStream_t)stream);
  if (e == hipSuccess && Y_bf16) {
    const size_t off = plan->off_act + ((size_t)(p.n_layers - 1) * plan->act_layer_elems + plan->a_x) * 2;
    e = hipMemcpyAsync(Y_bf16, ws + off, (size_t)p.M * p.d_model * 2, hipMemcpyDeviceToDevice, (hipStream_t)stream);
  }
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

int sgemm_chain_buffer(sgemm_plan plan, int layer, int which, size_t* offset, size_t* bytes) {
  if (!plan || !offset || !bytes) return SGEMM_ERR_INVALID_ARG;
  const sgemm_problem& p = plan->prob;
  if (p.kind == SGEMM_KIND_DECODER) {
    if (layer < 0 || layer >= p.n_layers || which < 0 || which > 4) return SGEMM_ERR_INVALID_ARG;
    const size_t q = (size_t)p.n_heads * p.head_dim, kv = (size_t)p.n_kv_heads * p.head_dim;
    const size_t offs[5] = {plan->a_h1, plan->a_h2, plan->a_x1, plan->a_a, plan->a_x};
    const size_t cols[5] = {q + 2 * kv, q, (size_t)p.d_model, (size_t)p.d_ff, (size_t)p.d_model};
    *offset = plan->off_act + ((size_t)layer * plan->act_layer_elems + offs[which]) * 2;
    *bytes = (size_t)p.M * cols[which] * 2;
    return SGEMM_OK;
  }
  if (p.kind != SGEMM_KIND_LAYERCHAIN) return SGEMM_ERR_INVALID_ARG;
  if (layer < 0 || layer >= p.n_layers || which < 0 || which > 3) return SGEMM_ERR_INVALID_ARG;
  const size_t offs[4] = {plan->a_h1, plan->a_h2, plan->a_a, plan->a_x};
  const size_t cols[4] = {(size_t)p.q_cols, (size_t)p.d_model, (size_t)p.d_ff, (size_t)p.d_model};
  *offset = plan->off_act + ((size_t)layer * plan->act_layer_elems + offs[which]) * 2;
  *bytes = (size_t)p.M * cols[which] * 2;
  return SGEMM_OK;
}

int sgemm_query_status(sgemm_plan plan, void* workspace, void* stream) {
  if (!plan || !workspace) return SGEMM_ERR_INVALID_ARG;
  if (hipSetDevice(plan->device) != hipSuccess) return SGEMM_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SGEMM_ERR_HIP;
  unsigned st = 0;
  if (hipMemcpy(&st, workspace, 4, hipMemcpyDeviceToHost) != hipSuccess) return SGEMM_ERR_HIP;
  if (st) {
    const unsigned zero = 0;
    if (hipMemcpy(workspace, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return SGEMM_ERR_HIP;
  }
  if (st & 1u) return SGEMM_ERR_TIMEOUT;
  if (st & 2u) return SGEMM_ERR_TOPOLOGY;  // work indexed by XCD would be duplicated or missing
  return SGEMM_OK;
}

const char* sgemm_status_string(int status) {
  switch (status) {
    case SGEMM_OK: return "ok";
    case SGEMM_ERR_INVALID_ARG: return "invalid argument";
    case SGEMM_ERR_UNSUPPORTED: return "unsupported problem";
    case SGEMM_ERR_HIP: return "HIP runtime error";
    case SGEMM_ERR_TIMEOUT: return "device wait timed out";
    case SGEMM_ERR_WORKSPACE: return "workspace error";
    case SGEMM_ERR_TOPOLOGY: return "workgroups did not map onto the XCDs as a rotated round-robin";
    default: return "unknown status";
  }
}

static std::string geo_json(const Geo& g) {
  char b[1024];
  std::snprintf(b, sizeof b,
                "{\"path\":\"%s\",\"M\":%d,\"K\":%d,\"N\":%d,\"ta\":%d,\"tb\":%d,\"waves\":%d,\"wpi\":%d,"
                "\"ksl\":%d,\"kss\":%d,\"TN\":%d,\"CB\":%d,\"Nx\":%d,\"NB\":%d,\"S\":%d,\"KS\":%d,"
                "\"steps\":%d,\"items\":%d,\"win\":%d,\"lds\":%d,\"stash_cap\":%d,\"paired\":%d,"
                "\"ring\":%d,\"mtiles\":%d,\"nfast\":%d,\"slots\":%d,\"xbuf\":%d,\"wpf\":%d,"
                "\"rr\":%d,\"mb\":%d,\"est_us\":%.3f}",
                g.path == 0 ? "dot2" : (g.path == 3 ? "kc" : (g.path >= 5 ? "lt" : "mfma")), g.M, g.K, g.N, g.ta, g.tb, g.waves, g.wpi, g.ksl, g.kss, g.TN,
                g.CB, g.Nx, g.NB, g.S, g.KS, g.steps, g.items, g.win, g.lds, g.stash_cap, g.paired, g.ring, g.mtiles,
                g.nfast, g.slots, g.xbuf, g.wpf, g.rr, g.mb, g.est_us);
  return b;
}

int sgemm_plan_describe(sgemm_plan plan, char* buf, size_t len) {
  if (!plan) return SGEMM_ERR_INVALID_ARG;
  std::string s = "{\"kind\":";
  s += plan->prob.kind == SGEMM_KIND_GEMM ? "\"gemm\"" : (plan->prob.kind == SGEMM_KIND_DECODER ? "\"decoder\"" : "\"layerchain\"");
  char b[256];
  std::snprintf(b, sizeof b,
                ",\"grid\":%d,\"workspace\":%zu,\"w_aux\":%u,\"sync\":\"%s\",\"stamps_offset\":%zu,",
                plan->grid, plan->ws_bytes, plan->w_aux, plan->sync == SYNC_XCD ? "xcd" : "agent",
                plan->off_stamps);
  s += b;
  if (plan->prob.kind == SGEMM_KIND_DECODER) {
    std::snprintf(b, sizeof b, "\"lds\":%d,\"chunks\":%d,\"attn_slices\":%d,", plan->dec_lds, plan->nchunk,
                  plan->attn_s);
    s += b;
  }
  if (plan->prob.kind == SGEMM_KIND_GEMM) {
    s += "\"stage\":" + geo_json(plan->geo);
  } else {
    s += "\"stages\":[";
    for (int i = 0; i < kChainStages; ++i) s += (i ? "," : "") + geo_json(plan->cg[i]);
    s += "]";
  }
  s += "}";
  if (buf && len) {
    std::strncpy(buf, s.c_str(), len - 1);
    buf[len - 1] = 0;
  }
  return (int)s.size() + 1;
}

int sgemm_device_check(int device) { return device_check(device); }

int sgemm_topology_probe(int* xcc_out, int n_wg, void* stream) {
  if (!xcc_out || n_wg < 1 || n_wg > 65536) return SGEMM_ERR_INVALID_ARG;
  return launch_topology(xcc_out, n_wg, (hipStream_t)stream) == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
}

int sgemm_read_probe(const void* src, size_t bytes, int pattern, unsigned* sink, int grid, void* stream) {
  if (!src || !sink || !aligned16(src) || ((uintptr_t)sink & 3u)) return SGEMM_ERR_INVALID_ARG;
  if (bytes < 16 || bytes % 16 || bytes >= kMaxOperand) return SGEMM_ERR_INVALID_ARG;
  if ((pattern != 0 && pattern != 1) || grid < 8 || grid > 4096 || grid % 8) return SGEMM_ERR_INVALID_ARG;
  return launch_stream_read(src, bytes, pattern, sink, grid, (hipStream_t)stream) == hipSuccess ? SGEMM_OK
                                                                                               : SGEMM_ERR_HIP;
}

}  // extern "C"
