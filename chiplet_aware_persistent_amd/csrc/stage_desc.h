// One GEMM "stage" as the device sees it: operands, the per-XCD column
// partition and the split-K decomposition chosen by the planner.  Plain POD,
// passed by value as a kernel argument (and as an array of them to the chain
// kernel).
#pragma once
#include <stdint.h>

namespace sg {

constexpr int kXcds = 8;            // XCDs (chiplets) of an MI355X in SPX mode
constexpr int kDot2KStep = 512;     // K values one dot2 wave step covers (64 lanes x 8)
constexpr int kMfmaKStep = 64;      // K values one MFMA wave step covers (2 x 32)
constexpr int kMaxWaves = 8;        // waves per workgroup (512 threads)
constexpr int kLoadsInFlight = 16;  // 16-byte weight loads per lane kept in flight

// Ring depth (k-steps in flight) of each path; steps per item are padded to a
// multiple of it.
constexpr int ring_depth_dot2(int g) { return g <= 1 ? 8 : (g <= 4 ? 4 : 2); }
// MFMA: 2 NT loads per lane and step.  One n-tile keeps 4 steps (8 loads) in
// flight, or 8 steps (16 loads) when `deep`; two n-tiles keep 4 steps.
constexpr int ring_depth_mfma(int nt, bool deep = false) {
  return nt == 1 ? (deep ? 8 : 4) : kLoadsInFlight / (2 * nt);
}
// MFMA steps per item are padded to this multiple of every ring depth above.
constexpr int step_pad_mfma(int nt) { return kLoadsInFlight / (2 * nt) > 2 ? kLoadsInFlight / (2 * nt) : 2; }

// Large-tile MFMA path (lt_device.h): four waves, 64-wide K steps; each
// step's 2 MW + 2 NW two-kilobyte operand blocks (16 rows x 64 K values) are
// fetched into registers several steps ahead, two whole-line loads per
// block, and written to one of two LDS buffers; the planner sizes the
// kernel's LDS with the same functions.
// Waves: 4 (2 x 2 over the tile) or 8 (2 x 4); MW x NW 16 x 16 tiles per wave.
constexpr int kLtKStep = 64;                // K values per step (two MFMA k-halves)
constexpr int lt_frags(int mw, int nw, int wv) { return 2 * mw + (wv / 2) * nw; }  // 2 KB blocks per step
constexpr int lt_loads_per_wave(int mw, int nw, int wv) { return (2 * lt_frags(mw, nw, wv) + wv - 1) / wv; }
// Steps in flight in registers: about 24 16-byte loads per lane, an even
// number from 2 to 8 (items are padded to a multiple of it).
constexpr int lt_reg_steps(int mw, int nw, int wv) {
  return (24 / lt_loads_per_wave(mw, nw, wv)) / 2 * 2 < 2 ? 2
         : ((24 / lt_loads_per_wave(mw, nw, wv)) / 2 * 2 > 8 ? 8 : (24 / lt_loads_per_wave(mw, nw, wv)) / 2 * 2);
}
constexpr int lt_lds_bytes(int mw, int nw, int wv) { return 2 * lt_frags(mw, nw, wv) * 2048; }

enum OutMode : int {
  OUT_F32 = 0,       // Y fp32
  OUT_BF16 = 1,      // Y bf16 (RNE)
  OUT_SILU_BF16 = 2, // paired gate/up tile: Y = bf16(silu(g) * u)
  OUT_BF16_F32 = 3   // Y bf16 and Y2 fp32 (the chain's last down projection)
};

enum SyncMode : int { SYNC_AGENT = 0, SYNC_XCD = 1 };

struct StageDesc {
  const uint16_t* X;   // activations, row-major [M][ldx]
  const uint16_t* W;   // weights, K-major [rows][K]
  void* Y;             // output, row-major [M][ldy]
  void* Y2;            // second output (OUT_BF16_F32), same layout, fp32
  float* part;         // split-K partials of this stage
  unsigned* ctr;       // split-K arrival counters of this stage (one per wave tile)
  int M, K, N;         // N = output columns (gate columns when paired)
  int ldx, ldy;
  int Nx;              // columns owned by one XCD (XCD x: [x*Nx, min(N,(x+1)*Nx)))
  int TN;              // columns per wave tile
  int wpi;             // waves per item: a workgroup runs waves/wpi item streams
  int ksl;             // K slices per item (MFMA): wpi = (wpi/ksl) column groups x ksl
  int kss;             // K values per slice (multiple of the k-step when ksl > 1)
  int CB;              // columns per item = (wpi / ksl) * TN
  int NB;              // column blocks per XCD
  int S;               // K splits
  int KS;              // K values per split (multiple of 8)
  int steps;           // wave k-steps per item (per K slice), padded to the ring depth
  int items;           // items per XCD = NB * S (ordered split-major)
  int ng;              // item streams (wave groups) per workgroup = waves / wpi
  int win;             // LDS window width (elements)
  int xrow;            // LDS row stride (elements)
  int red_off;         // LDS byte offset of the K-slice reduction buffer
  int stash_off;       // LDS byte offset of the output stash
  int stash_cap;       // items per owning wave whose results wait in LDS until the
                       // weight stream ends (the rest are stored at item end)
  int pair_off;        // paired: weight row offset of the up half
  int mtiles;          // MFMA: items per (split, column block), one 16-row m-tile each (1: all rows)
  int interleave;      // streams of a workgroup take every ng-th item of its range
  int rr;              // dot2, one K split: stream w of the XCD takes items w, w + streams, ...
  int nfast;           // m-tile items: column block fastest (the M-split order) instead of m-tile fastest
  int mode;            // OutMode
  int sync;            // SyncMode of the split-K arrival
  int check;           // single GEMM: claim (XCD, slot) at the end and latch a duplicate
  int xbuf;            // K-chunked MFMA path: bytes of one X chunk buffer (multiple of 1 KB)
  int nctr;            // split-K arrival counters of this stage (reset by the chain's last workgroup)
  int mb;              // K-chunked MFMA path: m-blocks of 16 MT rows per (split, column block) (0 or 1: one)
  int wpf;             // chain, dot2: steps of each wave's first item whose weights go to LDS before the wait
  int wpf_off;         // LDS byte offset of those weights (wave w: wpf * G kilobytes from wpf_off + w * that)
  const uint16_t* R;   // residual added to every output before its rounding (null: none), [M][ldy] bf16
  unsigned r_bytes;    // extent of R
  unsigned w_aux;      // cache-policy bits of the weight loads
  unsigned x_bytes, w_bytes, y_bytes, y2_bytes;  // operand extents (buffer bounds)
  unsigned part_bytes;                           // extent of the partial buffer
};

}  // namespace sg
