// The persistent layer chain kernel, shared by the translation units that
// instantiate it (MFMA stages in chain_kernel.hip, dot2 stages in
// chain_dot2.hip).
//
// Every projection of every layer in one launch.
//
// Per layer (Fleet reading note, sections 3f and 7b: gate and up are one
// concatenated GEMM whose result is SiLU-gated; a decoder layer's projections
// run back to back inside one persistent megakernel, section 2):
//   event 4l+0  h1 = bf16(x . Wq^T)
//   event 4l+1  h2 = bf16(h1 . Wo^T)
//   event 4l+2  a  = bf16(silu(g) * u), [g|u] = h2 . Wgu^T  (gate column j and
//               up column j are computed by the same wave, so the SiLU gate is
//               applied in the epilogue and only a is written)
//   event 4l+3  x' = bf16(a . Wdown^T)  (+ fp32 for the last layer)
//
// Completion of an event is published with two-level counters (Fleet reading
// note, section 2b flowchart (b) and section 3d): every workgroup bumps its
// XCD's counter L[x][e] (the 32 workgroups of an XCD share one L2, so no
// write-back is needed between them); the workgroup that brings L[x][e] to 32
// writes the XCD's L2 back (device-scope release) and bumps the global G[e].
// G[e] has one copy per consumer XCD, all eight bumped by one instruction
// of the releasing wave, so each copy is polled by 32 workgroups instead of
// one address by 256.  Consumers wait for their copy of G[e] to reach 8.  With
// SGEMM_F_SYNC_FLAT every workgroup does the release and bumps G[e] (target
// = grid), flowchart (a).
//
// With SGEMM_F_SCHEDULER (the per-XCD scheduler runtime of the Fleet reading
// note, sections 3b and 5 and the runtime layout figure of section 4) slot 0
// of each XCD runs no stage: it waits for each event's global counter and
// then releases the next task to the XCD's 31 workers by writing its id into
// their ready-task words (the per-worker last-ready-task id of section 11a,
// finding 4).  A worker polls only its own word; the stages' items are split
// over the 31 workers, and an XCD's last worker is the 31st to arrive.
//
// Before waiting, a workgroup already has the first weight steps of the next
// stage in flight (weights do not depend on the activations).  Every wait is
// bounded by a wall-clock budget; on expiry the time-out bit is latched in
// the status word and the workgroup stops, so a broken schedule ends the
// launch instead of hanging it.  The last workgroup to finish resets every
// counter for the next launch.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_device.h"
#include "kc_device.h"
#include "launch.h"

namespace sg {

static __device__ __forceinline__ unsigned long long now_ticks() { return wall_clock64(); }

// Wait until event e is complete (all producers published).  Executed by the
// whole workgroup; returns false when the wait timed out (here or elsewhere).
// Thread 0 of every workgroup polls its XCD's copy of the global counter with
// device-coherent loads.  With poll_leader, one leader per XCD (slot 0) polls it instead and,
// once it is complete, raises the XCD's flag, which the other 31 workgroups
// of the XCD poll (the per-XCD scheduler's polling role in the Fleet note,
// sections 2a and 3b, without a dedicated workgroup): fewer pollers share the
// counter's address, but the extra hop costs about a microsecond per stage
// on MI355X, more than the contention of 256 pollers does.
static __device__ __forceinline__ bool wait_event(const ChainArgs& a, int e, int xcd, int slot, int* sh_alive) {
  const int events = a.spl * a.n_layers;
  const unsigned* gc = a.gctr + (a.gcopies > 1 ? xcd * events : 0) + e;  // this XCD's copy
  const unsigned target = a.flat_sync ? gridDim.x : (unsigned)kXcds;
  const bool leader = slot == 0 || a.flat_sync || !a.poll_leader;
  if (threadIdx.x == 0) {
    unsigned* flag = a.xflag + xcd * events + e;
    int ok = 1;
    const unsigned long long t0 = now_ticks();
    for (;;) {
      bool done;
      if (a.sched) {
        // Released by the XCD's scheduler once event e is complete.
        done = __hip_atomic_load(a.ready + xcd * 32 + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
               (unsigned)(e + 1);
      } else if (leader) {
        done = __hip_atomic_load(gc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target;
      } else {
        // Device-scope read (it skips the CU's L1, which could hold a stale 0).
        done = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
      }
      if (done) break;
      if ((long long)(now_ticks() - t0) > a.spin_ticks ||
          (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout)) {
        __hip_atomic_fetch_or(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    // Acquire: with the producers' release (or, in scheduler mode, the
    // scheduler's acquire-release) it orders the stage's X reads after the
    // producers' writes.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (leader && ok && !a.flat_sync && a.poll_leader && !a.sched)
      __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sh_alive = ok;
  }
  __syncthreads();
  return *sh_alive != 0;
}

// Publish that this workgroup finished event e.
// The workgroup's stores are acknowledged by its XCD's L2 before its bump of
// L[x][e] (the fence keeps the compiler from moving them below the wait); the
// XCD's last workgroup writes that L2 back with a device-scope release before
// it bumps G[e], so the stores of all 32 workgroups reach memory before any
// consumer, which acquires after seeing G[e] == 8, reads them.
static __device__ __forceinline__ void signal_event(const ChainArgs& a, int e, int xcd, int nslots) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  wait_vm0();  // this wave's stores are acknowledged by L2
  __syncthreads();
  if (threadIdx.x < 64) {
    // Wave 0: lane 0 counts the workgroup in; lane c < gcopies bumps copy c.
    // (The lane index is opaque here so that the copies' addresses are not
    // hoisted out of the stage loop and kept in registers for the launch.)
    int lane = threadIdx.x;
    asm volatile("" : "+v"(lane));
    const int events = a.spl * a.n_layers;
    unsigned old = 0;
    if (!a.flat_sync && lane == 0)
      old = __hip_atomic_fetch_add(a.lctr + xcd * events + e, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.flat_sync || __builtin_amdgcn_readfirstlane(old) == (unsigned)(nslots - 1)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // write this XCD's L2 back
      if (lane < a.gcopies)
        __hip_atomic_fetch_add(a.gctr + lane * events + e, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Scheduler mode, slot 0 of XCD xcd (wave 0 only): for every event of the
// launch that has a successor, wait until all XCDs completed it, then write
// the successor's id into the ready-task words of the XCD's workers (one
// 128-byte line, lanes 1..nslots-1 at once).  The acquire-release fence
// between the two makes the producers' writes visible to a worker that
// acquires after reading its word.  Returns false if a wait timed out.
static __device__ __forceinline__ bool run_scheduler(const ChainArgs& a, int xcd, int nslots) {
  const int lane = threadIdx.x & 63;
  for (int e = a.e_begin; e + 1 < a.e_end; ++e) {
    int ok = 1;
    if (lane == 0) {
      const unsigned long long t0 = now_ticks();
      for (;;) {
        const unsigned* gc = a.gctr + (a.gcopies > 1 ? xcd * a.spl * a.n_layers : 0) + e;
        if (__hip_atomic_load(gc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)kXcds) break;
        if ((long long)(now_ticks() - t0) > a.spin_ticks ||
            (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout)) {
          __hip_atomic_fetch_or(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (!__shfl(ok, 0)) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
    if (lane >= 1 && lane < nslots)
      __hip_atomic_store(a.ready + xcd * 32 + lane, (unsigned)(e + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

static __device__ __forceinline__ void stamp(const ChainArgs& a, int e, int which) {
  if (a.stamps && threadIdx.x == 0) {
    const int events = a.spl * a.n_layers;
    a.stamps[((size_t)blockIdx.x * events + e) * 2 + which] = now_ticks();
  }
}

// PATH 1: MFMA stages with A = MT m-tiles and B = NT n-tiles (the paired
// gate_up stage uses two).  PATH 0 (M < 16): dot2 stages with A = M rows and
// B = G weight rows per wave (gate_up: G/2 gate and G/2 up rows).  PATH 3:
// K-chunked MFMA stages (kc_device.h) with A = MT, B = 10 NTW_u + NTW_p tiles
// per item in the unpaired and the paired (gate_up) stages.
template <int PATH, int A, int B>
__global__ __launch_bounds__(512) void k_chain(ChainArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ int sh_alive;
  __shared__ int sh_last;
  const int xcd = xcd_of_wg(a.status);
  const int slot = blockIdx.x >> 3;
  const int nslots = gridDim.x >> 3;
  // Each workgroup claims its (XCD, slot) pair.  A pair claimed twice (or a
  // slot past 31) means the dispatch was not a rotated round-robin, and the
  // XCD-local counters would be wrong: recorded as a topology error.
  if (threadIdx.x == 0) {
    const unsigned bit = slot < 32 ? 1u << slot : 0u;
    const unsigned old = __hip_atomic_fetch_or(a.claim + xcd, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bit == 0u || (old & bit))
      __hip_atomic_fetch_or(a.status, kStatusTopology, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The scheduler (scheduler mode, slot 0) runs no stage; its other waves
  // go straight to the final barrier.
  const bool scheduler = a.sched && slot == 0;
  if (scheduler && threadIdx.x < 64) run_scheduler(a, xcd, nslots);
  // Workers: the stages' items are split over wn workgroups, wslot is ours.
  const int wslot = a.sched ? slot - 1 : slot;
  const int wn = a.sched ? nslots - 1 : nslots;
  bool alive = !scheduler;
  // Events e = 4 l + s of this launch, in order (all of them unless the
  // per-stage ablation splits the chain into launches).  The stage loop has a
  // compile-time s, so each stage's descriptor is selected statically.
  for (int l = a.e_begin >> 2; 4 * l < a.e_end && alive; ++l) {
    uint16_t* act = a.act + (size_t)l * a.act_layer_elems;
    const uint16_t* xin = l == 0 ? a.x0 : a.act + (size_t)(l - 1) * a.act_layer_elems + a.off_x;
    for (int s = 0; s < kChainStages && alive; ++s) {
      const int e = 4 * l + s;
      if (e < a.e_begin || e >= a.e_end) continue;  // another launch runs it
      StageDesc d = a.st[s];
      if (s == 0) { d.X = xin; d.W = a.wq[l]; d.Y = act + a.off_h1; }
      if (s == 1) { d.X = act + a.off_h1; d.W = a.wo[l]; d.Y = act + a.off_h2; }
      if (s == 2) { d.X = act + a.off_h2; d.W = a.wgu[l]; d.Y = act + a.off_a; }
      if (s == 3) {
        d.X = act + a.off_a; d.W = a.wdown[l]; d.Y = act + a.off_x;
        if (l == a.n_layers - 1) { d.mode = OUT_BF16_F32; d.Y2 = a.y_f32; }
      }
      auto hook = [&]() -> bool {
        // The launch's first event has its X complete (the previous launch, or the input).
        const bool ok = e == a.e_begin ? true : wait_event(a, e - 1, xcd, slot, &sh_alive);
        stamp(a, e, 0);
        return ok;
      };
      // Every workgroup runs the hook (the wait), also one without items here.
      if constexpr (PATH == 3) {
        if (s == 2) {
          alive = mfma_kc_stage<A, B % 10, true, kAuxNt, decltype(hook), true>(d, lds, xcd, wslot, wn, hook);
        } else {
          alive = mfma_kc_stage<A, B / 10, false, kAuxNt, decltype(hook), true>(d, lds, xcd, wslot, wn, hook);
        }
      } else if constexpr (PATH == 1) {
        // Up to two m-tiles (M <= 32) keep the deeper ring: across the stage
        // barriers it measured faster there, the shallow one at M = 64.
        if (s == 2) {
          alive = mfma_stage<A, 2, true, kAuxNt, (A <= 2)>(d, lds, xcd, wslot, wn, hook);
        } else {
          alive = mfma_stage<A, B, false, kAuxNt, (A <= 2)>(d, lds, xcd, wslot, wn, hook);
        }
      } else {
        if (s == 2) {
          alive = dot2_stage<A, B, kAuxNt, true>(d, lds, xcd, wslot, wn, hook);
        } else {
          alive = dot2_stage<A, B, kAuxNt, false>(d, lds, xcd, wslot, wn, hook);
        }
      }
      if (!alive) break;
      if (a.stamps) __syncthreads();  // the stamp marks the end of the workgroup's last wave
      stamp(a, e, 1);
      if (e + 1 < a.e_end) signal_event(a, e, xcd, wn);  // the launch's last event has no waiter
      __syncthreads();  // LDS window reuse by the next stage
    }
  }
  // Finish: the last workgroup resets all counters for the next launch.
  // Every counter is touched only by device-scope atomics, and vmcnt(0) has
  // seen each of this workgroup's complete before it counts itself done, so
  // no release (an L2 write-back per workgroup) precedes the done count: no
  // other workgroup reads this one's data after this point, and the end of
  // the kernel writes it back.
  wait_vm0();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = old == gridDim.x - 1;
    if (sh_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (sh_last) {
    // Only this launch's events [e_begin, e_end) and their stages touched
    // counters; every other event's counters are still zero.
    const int events = a.spl * a.n_layers;
    const int ne = a.e_end - a.e_begin;
    for (int i = threadIdx.x; i < a.gcopies * ne; i += blockDim.x) {
      const int c = i / ne;
      a.gctr[c * events + a.e_begin + (i - c * ne)] = 0u;
    }
    for (int i = threadIdx.x; i < kXcds * ne; i += blockDim.x) {
      const int x = i / ne;
      const int e = a.e_begin + (i - x * ne);
      a.lctr[x * events + e] = 0u;
      a.xflag[x * events + e] = 0u;
    }
    if (threadIdx.x < kXcds) a.claim[threadIdx.x] = 0u;
    if (threadIdx.x < kXcds * 32) a.ready[threadIdx.x] = 0u;
    for (int s = 0; s < kChainStages; ++s) {
      bool used = ne >= kChainStages;
      for (int e = a.e_begin; e < a.e_end && !used; ++e) used = (e & 3) == s;
      if (!used) continue;
      const int n = a.st[s].nctr;
      for (int i = threadIdx.x; i < n; i += blockDim.x) a.st[s].ctr[i] = 0u;
    }
    wait_vm0();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

typedef void (*ChainKernel)(ChainArgs);

// dot2 instantiations (M = 1..15, G = 2 or 4), null when absent.
ChainKernel chain_kernel_dot2(int m, int g);
// K-chunked instantiations (MT, 10 NTW_u + NTW_p), null when absent.
ChainKernel chain_kernel_kc(int mt, int code);

}  // namespace sg
