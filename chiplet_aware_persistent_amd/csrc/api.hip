// C ABI of libsgemm.so: validation, planning and launches.  See include/sgemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
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
constexpr int kLdsMax = 160 * 1024;     // LDS budget of one workgroup (one per CU; 160 KB/CU)
constexpr size_t kMaxOperand = (size_t)1 << 31;  // buffer extents are 31-bit here
constexpr int kWgPerXcd = 32;           // one workgroup per CU, 32 CUs per XCD

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Decomposition of one GEMM stage (see gemm_device.h for how it is executed).
struct Geo {
  int path = 0;        // 0 dot2, 1 MFMA
  int M = 0, K = 0, N = 0;
  int ta = 0, tb = 0;  // template parameters: dot2 (M, G); MFMA (MT, NT)
  int waves = 8, wpi = 8, ng = 1, TN = 0, CB = 0, Nx = 0, NB = 0, S = 1, KS = 0, steps = 0, items = 0;
  int ksl = 1, kss = 0;
  int win = 0, xrow = 0, lds = 0, red_off = 0, stash_off = 0, stash_cap = 0;
  int paired = 0, pair_off = 0;
  int ring = 0;    // ring depth (k-steps in flight per wave)
  int mtiles = 1;  // m-tile items (ablation): items per (split, column block), m-tile fastest
  int slots = 32;  // workgroups per XCD that share the items (31 with a scheduler workgroup)
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
  g.stash_cap = std::max(0, std::min(per_stream, (kLdsMax - g.stash_off) / (owners * tile_bytes)));
  g.lds = g.stash_off + owners * g.stash_cap * tile_bytes;
  const int vals = g.path == 0 ? g.tb * g.M : g.tb * g.ta * 256;
  g.ctr_count = (size_t)kXcds * g.NB * g.wpi * g.mtiles;
  g.part_floats = g.S > 1 ? g.ctr_count * (size_t)g.S * vals : 0;
  if (g.stash_off > kLdsMax) return false;
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
              int ksl_o, const Cost& cost, int wpi_o = 0, bool mtile_items = false, int slots = kWgPerXcd) {
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
        if (mtile_items) {  // one 16-row m-tile per item, one wave per item
          if (wpi != 1 || ksl != 1) continue;
          g.mtiles = g.ta;
          g.ta = 1;
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
  long long spin_ticks = 0;
};

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int validate_gemm(const sgemm_problem& p) {
  if (p.M < 1 || p.K < 8 || p.N < 1) return SGEMM_ERR_INVALID_ARG;
  if (p.K % 8 != 0) return SGEMM_ERR_INVALID_ARG;
  if (p.out_dtype != SGEMM_OUT_F32 && p.out_dtype != SGEMM_OUT_BF16) return SGEMM_ERR_INVALID_ARG;
  if (p.M > 64) return SGEMM_ERR_UNSUPPORTED;
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

  sgemm_plan_s* pl = new (std::nothrow) sgemm_plan_s();
  if (!pl) return SGEMM_ERR_INVALID_ARG;
  pl->prob = p;
  pl->device = device;
  pl->w_aux = (p.flags & SGEMM_F_W_CACHED) ? 0u : ((p.flags & SGEMM_F_W_SC1) ? 18u : 2u);
  pl->sync = (p.flags & SGEMM_F_SYNC_AGENT) ? SYNC_AGENT : SYNC_XCD;

  size_t cur = kCtl;
  if (p.kind == SGEMM_KIND_GEMM) {
    if (p.flags & SGEMM_F_SCHEDULER) { delete pl; return SGEMM_ERR_UNSUPPORTED; }  // a chain runtime
    int rc = validate_gemm(p);
    if (rc != SGEMM_OK) { delete pl; return rc; }
    const bool mti = (p.flags & SGEMM_F_MTILE_ITEMS) != 0;
    if (mti && (p.flags & SGEMM_F_FORCE_DOT2)) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    const int path = mti ? 1 : choose_path(p);
    if ((path == 0 || mti) && k_o > 1) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    if (!plan_geo(pl->geo, p.M, p.K, p.N, path, 0, tn_o, s_o, w_o, k_o, kCostGemm, 0, mti)) {
      delete pl;
      return SGEMM_ERR_UNSUPPORTED;
    }
    layout_stage_ws(cur, pl->geo, pl->off_ctr, pl->off_part);
  } else if (p.kind == SGEMM_KIND_LAYERCHAIN) {
    if (p.flags & (SGEMM_F_W_CACHED | SGEMM_F_W_SC1 | SGEMM_F_MTILE_ITEMS)) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    const bool sched = (p.flags & SGEMM_F_SCHEDULER) != 0;
    if (sched && (p.flags & (SGEMM_F_SYNC_FLAT | SGEMM_F_POLL_LEADER))) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    const int slots = sched ? kWgPerXcd - 1 : kWgPerXcd;  // the scheduler workgroup takes no items
    if (p.M < 1 || p.n_layers < 1 || p.d_model < 8 || p.q_cols < 8 || p.d_ff < 8)
      { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if (p.d_model % 8 || p.q_cols % 8 || p.d_ff % 8) { delete pl; return SGEMM_ERR_INVALID_ARG; }
    if (p.M > 64 || p.n_layers > kMaxLayers) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
    if ((size_t)2 * p.d_ff * p.d_model * 2 >= kMaxOperand) { delete pl; return SGEMM_ERR_UNSUPPORTED; }
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
    for (int waves = 8; waves >= 4; waves -= 4) {
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
    // Re-layout with the final geometries.
    cur = kCtl;
    for (int s = 0; s < kChainStages; ++s) layout_stage_ws(cur, pl->cg[s], pl->c_ctr[s], pl->c_part[s]);
    const int events = kChainStages * p.n_layers;
    pl->off_lctr = cur;
    cur = round_up(cur + (size_t)kXcds * events * 4, 256);
    pl->off_gctr = cur;
    cur = round_up(cur + (size_t)events * 4, 256);
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
  d.w_aux = w_aux;
  d.sync = sync;
  return d;
}

int sgemm_run(sgemm_plan plan, const void* X, const void* W, void* Y, void* workspace, void* stream) {
  if (!plan || !X || !W || !Y || !workspace) return SGEMM_ERR_INVALID_ARG;
  if (plan->prob.kind != SGEMM_KIND_GEMM) return SGEMM_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || !aligned16(workspace))
    return SGEMM_ERR_INVALID_ARG;
  const sgemm_problem& p = plan->prob;
  const Geo& g = plan->geo;
  StageDesc d = stage_desc(g, plan->w_aux, plan->sync);
  char* ws = (char*)workspace;
  d.X = (const uint16_t*)X;
  d.W = (const uint16_t*)W;
  d.Y = Y;
  d.Y2 = nullptr;
  d.ldx = p.K;
  d.ldy = p.N;
  d.mode = p.out_dtype == SGEMM_OUT_F32 ? OUT_F32 : OUT_BF16;
  d.part = (float*)(ws + plan->off_part);
  d.part_bytes = (unsigned)(g.part_floats * 4);
  d.ctr = (unsigned*)(ws + plan->off_ctr);
  d.x_bytes = (unsigned)((size_t)p.M * p.K * 2);
  d.w_bytes = (unsigned)((size_t)p.N * p.K * 2);
  d.y_bytes = (unsigned)((size_t)p.M * p.N * (p.out_dtype == SGEMM_OUT_F32 ? 4 : 2));
  d.y2_bytes = 0;
  if (hipSetDevice(plan->device) != hipSuccess) return SGEMM_ERR_HIP;
  hipError_t e = launch_gemm(d, g.mtiles > 1 ? 2 : g.path, g.ta, g.tb, plan->grid, g.waves * 64, g.lds, (unsigned*)ws,
                             (hipStream_t)stream);
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_HIP;
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
  a.act_layer_elems = plan->act_layer_elems;
  a.off_h1 = plan->a_h1; a.off_h2 = plan->a_h2; a.off_a = plan->a_a; a.off_x = plan->a_x;
  a.flat_sync = (p.flags & SGEMM_F_SYNC_FLAT) ? 1 : 0;
  a.poll_leader = (p.flags & SGEMM_F_POLL_LEADER) ? 1 : 0;
  a.sched = (p.flags & SGEMM_F_SCHEDULER) ? 1 : 0;
  a.spin_ticks = plan->spin_ticks;
  a.path = plan->cg[0].path;
  a.mt = plan->cg[0].ta;
  a.nt_q = plan->cg[0].tb; a.nt_o = plan->cg[1].tb; a.nt_d = plan->cg[3].tb;
  int lds = 0;
  for (int s = 0; s < kChainStages; ++s) lds = std::max(lds, plan->cg[s].lds);
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

int sgemm_chain_buffer(sgemm_plan plan, int layer, int which, size_t* offset, size_t* bytes) {
  if (!plan || !offset || !bytes || plan->prob.kind != SGEMM_KIND_LAYERCHAIN) return SGEMM_ERR_INVALID_ARG;
  const sgemm_problem& p = plan->prob;
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
  char b[512];
  std::snprintf(b, sizeof b,
                "{\"path\":\"%s\",\"M\":%d,\"K\":%d,\"N\":%d,\"ta\":%d,\"tb\":%d,\"waves\":%d,\"wpi\":%d,"
                "\"ksl\":%d,\"kss\":%d,\"TN\":%d,\"CB\":%d,\"Nx\":%d,\"NB\":%d,\"S\":%d,\"KS\":%d,"
                "\"steps\":%d,\"items\":%d,\"win\":%d,\"lds\":%d,\"stash_cap\":%d,\"paired\":%d,"
                "\"ring\":%d,\"mtiles\":%d,\"slots\":%d,\"est_us\":%.3f}",
                g.path == 0 ? "dot2" : "mfma", g.M, g.K, g.N, g.ta, g.tb, g.waves, g.wpi, g.ksl, g.kss, g.TN,
                g.CB, g.Nx, g.NB, g.S, g.KS, g.steps, g.items, g.win, g.lds, g.stash_cap, g.paired, g.ring, g.mtiles, g.slots, g.est_us);
  return b;
}

int sgemm_plan_describe(sgemm_plan plan, char* buf, size_t len) {
  if (!plan) return SGEMM_ERR_INVALID_ARG;
  std::string s = "{\"kind\":";
  s += plan->prob.kind == SGEMM_KIND_GEMM ? "\"gemm\"" : "\"layerchain\"";
  char b[256];
  std::snprintf(b, sizeof b,
                ",\"grid\":%d,\"workspace\":%zu,\"w_aux\":%u,\"sync\":\"%s\",\"stamps_offset\":%zu,",
                plan->grid, plan->ws_bytes, plan->w_aux, plan->sync == SYNC_XCD ? "xcd" : "agent",
                plan->off_stamps);
  s += b;
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
