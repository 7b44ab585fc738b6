// Dependency waits and A-operand variants shared by the chain kernels.
#pragma once

#include "gemm_tile.h"

namespace tls {

// Dense row-major A operand (ROWS rows per tile) with nothing to fix.
template <class T, int ROWS = T::BM>
struct PlainRows : RowMajorRows<T, ROWS, kAuxNone>, NoFix {};

// Dense row-major A operand under the sentinel handoff.
template <class T>
using SentinelRows = SentinelFix<RowMajorRows<T, T::BM, kAuxNone>>;

// Wave-level wait for a set of monotone flags that must all be reached.
// `lane_ok()` loads this lane's share of the flags and says whether all of
// them are reached.  One pass over every lane, then, while some lane still
// misses a flag, only the first such lane re-polls (one load per round, with
// back-off), and once its flags are reached the lanes still missing reload
// once.  Waiting workgroups then put one coherent load per round on the
// fabric instead of one per flag, which matters while the producers they wait
// for still run.  Called by the 64 lanes of one wave; returns the same value
// on all of them (false: poll limit or abort).
template <class LANE_OK>
__device__ __forceinline__ bool wave_wait_all(LANE_OK&& lane_ok, uint32_t limit, Ctl* ctl) {
  const int lane = threadIdx.x & 63;
  bool done = lane_ok();
  uint64_t miss = __ballot(!done);
  for (uint32_t it = 0; miss != 0ull; ++it) {
    if (it >= limit) return false;
    if ((it & 63u) == 63u && ld_relaxed_agent(&ctl->abort)) return false;
    poll_pause(it);
    const int first = __builtin_ctzll(miss);
    if (lane == first) done = lane_ok();
    if ((__ballot(done) >> first) & 1ull) {
      if (!done) done = lane_ok();
    }
    miss = __ballot(!done);
  }
  return true;
}

struct TileSyncWait {
  const uint32_t* flags;  // first flag of the producer row
  int steps_per_tile;     // K steps per producer column tile
  int ntiles;             // producer column tiles
  uint32_t epoch;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ready;
  int ready;   // producer tiles [0, ready) of the row are known complete and acquired
  bool light;  // light acquire (see acquire_after_poll)
  int kt0;     // absolute K step of the loop's step 0 (K splits)
  static constexpr bool kStepWaits = true;
  // Every producer tile of the row is known complete: no later step waits.
  __device__ __forceinline__ bool all_ready() const { return ready >= ntiles; }
  __device__ __forceinline__ bool before(int ktl) {
    const int kt = ktl + kt0;
    if (kt % steps_per_tile && ktl != 0) return true;
    const int j = kt / steps_per_tile;
    if (j < ready) return true;
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int idx = j + lane;
      int got = -1;
      // One pass over the window [j, j + 64): the ready prefix.  While tile j
      // itself is missing, lane 0 alone re-polls its flag (one load per
      // round); once it is set, one more pass measures the prefix.
      bool full = true;
      for (uint32_t it = 0;; ++it) {
        if (full) {
          const bool ok =
              idx < ntiles && reached(ld_relaxed_agent(flags + idx * kFlagStride), epoch);
          const uint64_t m = __ballot(ok);
          const int run = (m == ~0ull) ? 64 : __builtin_ctzll(~m);
          if (run > 0) {
            got = j + run;
            break;
          }
          full = false;
        } else {
          const bool ok = lane == 0 && reached(ld_relaxed_agent(flags + j * kFlagStride), epoch);
          if (__ballot(ok) & 1ull) {
            full = true;
            continue;
          }
        }
        if (it >= limit) break;
        if ((it & 63u) == 63u && ld_relaxed_agent(&ctl->abort)) break;
        poll_pause(it);
      }
      if (lane == 0) {
        if (got >= 0)
          acquire_after_poll(light);
        else
          record_timeout(ctl, item, 1u);
        *s_ready = got;
      }
    }
    wg_barrier();
    ready = *s_ready;
    return ready >= 0;
  }
};

struct RowSyncWait {
  const uint32_t* counter;
  uint32_t target;
  uint32_t limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ok;
  bool light;  // light acquire (see acquire_after_poll)
  // Waits only before step 0 (the prologue): nothing left in the main loop.
  __device__ __forceinline__ bool all_ready() const { return true; }
  __device__ __forceinline__ bool before(int kt) {
    if (kt != 0) return true;
    if (threadIdx.x == 0) {
      const bool ok = poll_reached(counter, target, limit, ctl, light);  // acquires on success
      if (!ok) record_timeout(ctl, item, 1u);
      *s_ok = ok ? 1 : 0;
    }
    wg_barrier();
    return *s_ok != 0;
  }
};

// TileSync wait for a whole producer row before step 0: the flags of all of
// its tiles (each posted by its own producer tile), polled by wave 0's lanes
// in parallel, one acquire for all; no wait code in the main loop.  For
// consumers that need the whole row anyway (the attention softmax) or whose
// main loop cannot hold a per-step wait without spilling.
struct TileRowWait {
  const uint32_t* flags;  // first flag of the producer row
  int ntiles;             // producer tiles of the row
  uint32_t epoch, limit;
  Ctl* ctl;
  uint32_t item;
  int* s_ok;
  bool light;  // light acquire (see acquire_after_poll)
  __device__ __forceinline__ bool all_ready() const { return true; }
  __device__ __forceinline__ bool before(int kt) {
    if (kt != 0) return true;
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const bool ok = wave_wait_all(
          [&]() {
            bool mine = true;
            for (int j = lane; j < ntiles && mine; j += 64)
              mine = reached(ld_relaxed_agent(flags + j * kFlagStride), epoch);
            return mine;
          },
          limit, ctl);
      if (lane == 0) {
        if (ok)
          acquire_after_poll(light);
        else
          record_timeout(ctl, item, 1u);
        *s_ok = ok ? 1 : 0;
      }
    }
    wg_barrier();
    return *s_ok != 0;
  }
};

// Trace hook around any waiter: thread 0 notes when the item's first
// dependency wait (step 0) returned.  s_tready is null when not tracing.
template <class W>
struct TracedWait {
  static constexpr bool kStepWaits = StepWaits<W>::value;
  W& w;
  uint64_t* s_tready;
  __device__ __forceinline__ bool all_ready() const { return w.all_ready(); }
  __device__ __forceinline__ bool before(int kt) {
    const bool ok = w.before(kt);
    if (kt == 0 && s_tready != nullptr && threadIdx.x == 0) *s_tready = now_rt();
    return ok;
  }
};

}  // namespace tls
