// Host-side entry points of the kernel translation units, used by the C ABI.
#pragma once
#include <hip/hip_runtime.h>

#include "stage_desc.h"

namespace sg {

constexpr int kMaxLayers = 64;
constexpr int kChainStages = 4;  // Q, O, gate_up (paired, SiLU-gated), down

struct ChainArgs {
  StageDesc st[kChainStages];          // operands other than W/X/Y are filled per layer
  const uint16_t* wq[kMaxLayers];
  const uint16_t* wo[kMaxLayers];
  const uint16_t* wgu[kMaxLayers];
  const uint16_t* wdown[kMaxLayers];
  const uint16_t* x0;                  // [M][d] bf16
  uint16_t* act;                       // per-layer activations, see layout below
  float* y_f32;                        // last layer's down projection, fp32
  uint16_t* y_bf16;                    // its bf16 rounding (may be null)
  unsigned* status;                    // workspace word 0
  unsigned* lctr;                      // [kXcds][events] intra-XCD event counters
  unsigned* gctr;                      // [gcopies][events] global event counters (copy x polled by XCD x)
  unsigned* xflag;                     // [kXcds][events] per-XCD 'event seen' flags
  unsigned* done;                      // workgroups finished (reset by the last one)
  unsigned* claim;                     // [kXcds] slots claimed per XCD (reset by the last one)
  unsigned* ready;                     // [kXcds][32] scheduler mode: last task id released to each slot
  unsigned long long* stamps;          // [grid][events][2] or null
  int n_layers, M, d, q, dff;
  size_t act_layer_elems;              // bf16 elements per layer of activations
  size_t off_h1, off_h2, off_a, off_x; // element offsets inside one layer's block
  int flat_sync;                       // every workgroup publishes globally
  int poll_leader;                     // one workgroup per XCD polls and raises the XCD's flag
  int sched;                           // slot 0 of each XCD schedules, slots 1..31 work
  long long spin_ticks;                // watchdog budget (wall-clock ticks, 100 MHz)
  int gcopies;                         // copies of each global counter: 8 (one per consumer XCD) or 1
  int path;                            // 1: MFMA stages, 0: dot2 stages (M < 16)
  int mt, nt_q, nt_o, nt_d;            // template parameters: MFMA (MT, NT); dot2 (M in mt, G in nt_*); K-chunked: code in nt_q
  int e_begin, e_end;                  // events this launch runs: [e_begin, e_end)
  int spl;                             // stages (events) per layer: 4 (chain), 5 (decoder)
  // Decoder layer only (5 stages: QKV with the attention norm, attention,
  // O with the residual, gate_up with the MLP norm, down with the residual).
  const uint16_t* wnorm;               // [layers][2][d] bf16: attention and MLP RMSNorm weights
  const uint16_t* kc;                  // [layers][M][Hkv][T][hd] bf16 cached keys
  const uint16_t* vc;                  // same, values
  float* apart;                        // attention slice results [M][Hkv][slices][grp][hd + 2]
  unsigned* actr;                      // attention slice arrival counters [M][Hkv]
  int Hq, Hkv, hd, T, pc, nchunk;      // heads, head dim, cached positions, positions per chunk, chunks
  int attn_s;                          // attention slices (workgroups) per (sequence, head) pair, 1..8
  float eps;                           // RMSNorm epsilon
  int norm_off;                        // LDS byte offset of the RMSNorm factors (M floats)
  size_t off_qkv, off_o, off_x1;       // decoder: element offsets of qkv, o and x1 in a layer's block
};

bool gemm_variant_exists(int path, int a, int b);
hipError_t launch_gemm(const StageDesc& d, int path, int a, int b, int grid, int block, int lds,
                       unsigned* status, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_topology(int* out, int n, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, int pattern, unsigned* sink, int grid,
                              hipStream_t stream);

bool chain_variant_exists(int path, int a, int b);  // MFMA (MT, NT) or dot2 (M, G)
hipError_t launch_chain(const ChainArgs& a, int grid, int block, int lds, hipStream_t stream);
bool decoder_variant_exists(int path, int a, int b);
hipError_t launch_decoder(const ChainArgs& a, int grid, int block, int lds, hipStream_t stream);

}  // namespace sg
