// gfx950 device primitives: vector types, buffer loads/stores, agent-scope
// posts and acquires, bounded polling with a watchdog, activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace tls {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

#define TLS_LDS_AS __attribute__((address_space(3)))

// Cache-policy bits of buffer instructions on gfx950: sc1 makes a load
// coherent at agent scope (it cannot return a line another XCD's L2 still
// holds dirty or that this XCD's L2 holds stale); it is what the compiler
// emits for a relaxed agent-scope atomic load.
constexpr int kAuxNone = 0;
constexpr int kAuxAgent = 16;

// Raw buffer resource over [base, base + bytes).  Loads past the end return
// zero and stores past the end are dropped, which makes ragged row tiles safe.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The two kinds of global store of the chain kernels; every global store of
// tile data goes through one of these four helpers.
//
// publish16/publish8: data that another workgroup reads inside the same
// launch once a readiness flag (or a split arrival) says it is complete:
// intermediates (Z, scores, XQKV, XDot), split partials, a refilled sentinel
// slot.  Always device-scope (sc1): the store goes through the XCD's L2 to
// the level every XCD reads, and s_waitcnt vmcnt(0) counts it complete only
// then, which is what lets a relaxed post after a drain publish it (see
// post_store) and lets a consumer on another XCD read it without a release
// write-back of the producer's L2.
//
// store_out16/store_out8: results that no wave of the launch reads (Y, O):
// ordinary stores, made visible by the end of the kernel.
__device__ __forceinline__ void publish16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kAuxAgent);
}
__device__ __forceinline__ void publish8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kAuxAgent);
}
__device__ __forceinline__ void store_out16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kAuxNone);
}
__device__ __forceinline__ void store_out8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kAuxNone);
}

// Wait until every vector memory operation this wave issued has completed
// (stores acknowledged by L2).  __syncthreads() alone does not do this.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Readiness flags.  Post: every wave drains its device-scope stores, the
// workgroup meets at a barrier, then one lane updates the flag with a relaxed
// agent-scope atomic (post_store / post_add below: the stores themselves are
// what makes the tile visible to every XCD).  Wait: one lane polls with
// relaxed agent-scope loads, then an agent-scope ACQUIRE (invalidates stale
// lines in this CU/XCD, or its light form), then the workgroup barrier.  This
// is the semaphore pair of the cuSync paper, section "Synchronization
// Implementation" (post: barrier, fence, increment; wait: first thread spins,
// others wait at a barrier), with the fences chosen for the gfx950 memory
// model.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ld_relaxed_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire_agent() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Post of published data.  Producers store everything a flag publishes
// (intermediate tiles, split partials) with device-scope stores (the sc1 cache
// policy): the same instruction the compiler emits for a relaxed agent-scope
// atomic store, written through the XCD's L2 to the level every XCD reads,
// and counted complete by s_waitcnt vmcnt(0) only once it is there.  Every
// wave drains its stores and the workgroup meets at a barrier before one lane
// posts, so the flag itself is a relaxed agent-scope atomic after one more
// local drain.  The agent-scope release would add a write-back of every dirty
// line of the XCD's L2, whoever wrote it (consumer outputs included), a cost
// that grows with the number of posts (15-17 % of the attention chain's time
// with one post per score row).
__device__ __forceinline__ void post_store(uint32_t* p, uint32_t v) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void post_add(uint32_t* p, uint32_t v) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Arrival on a counter that publishes this workgroup's drained device-scope
// stores and, for the one arrival that completes it, acquires everyone
// else's (full agent-scope acquire: the arriving workgroup may hold stale
// lines of a reused buffer).  Returns the count before this arrival.
__device__ __forceinline__ uint32_t arrive_agent(uint32_t* p, uint32_t target) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint32_t before = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (before + 1u == target) fence_acquire_agent();
  return before;
}

// Acquire after a successful poll.  The full form is the agent-scope acquire
// of the AMDGPU memory model (invalidates this CU's L1 and the XCD's L2).  The
// light form only orders the poll before the loads that follow.  It suffices
// when (a) every cache line the consumer reads after the flag lies wholly in
// data that flag published and (b) no wave of the launch read those lines
// before they were published: the dispatch invalidated every cache when the
// launch began, so the first touch of such a line on any XCD fetches the
// bytes the producer's drained device-scope stores put there.  Producers and
// consumers of the chains satisfy (b) by construction (only consumers read the
// intermediate,
// only after its flag); the host asks for the light form only when the
// intermediate is 128-byte aligned, which gives (a) since every tile then
// covers whole 128-byte lines.
__device__ __forceinline__ void acquire_after_poll(bool light) {
  if (light)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    fence_acquire_agent();
}

// Pause between two polls of a readiness flag: exponential back-off from one
// short sleep (about 128 cycles) up to kPollPauseCap of them, so that waiting
// workgroups do not flood the memory fabric with coherent loads while the
// producers run, yet notice a posted flag within about half a microsecond.
constexpr uint32_t kPollPauseCap = 8;
__device__ __forceinline__ void poll_pause(uint32_t it) {
  const uint32_t n = it < 3u ? (1u << it) : kPollPauseCap;
  for (uint32_t k = 0; k < n; ++k) __builtin_amdgcn_s_sleep(2);
}

// Wrap-safe "value has reached target" for monotone u32 counters.
__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) {
  return (int32_t)(v - target) >= 0;
}

// Record the first watchdog expiry of a launch and ask every workgroup to stop.
__device__ __forceinline__ void record_timeout(Ctl* ctl, uint32_t item, uint32_t kind) {
  uint32_t expected = kStatusOk;
  if (__hip_atomic_compare_exchange_strong(&ctl->status, &expected, (uint32_t)kStatusTimeout,
                                           __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(&ctl->status_item, item, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctl->status_kind, kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_store(&ctl->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll until *p reaches target (then acquire) or the limit / an abort ends
// the wait.  Called by one lane.  Every iteration sleeps briefly so the
// spinning wave leaves issue slots to co-resident waves.
__device__ __forceinline__ bool poll_reached(const uint32_t* p, uint32_t target, uint32_t limit,
                                             const Ctl* ctl, bool light) {
  for (uint32_t it = 0;; ++it) {
    if (reached(ld_relaxed_agent(p), target)) {
      acquire_after_poll(light);
      return true;
    }
    if (it >= limit) return false;
    if ((it & 63u) == 63u && ld_relaxed_agent(&ctl->abort)) return false;
    poll_pause(it);
  }
}

// ---------------------------------------------------------------------------
// fp16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f16_bits(f16 h) { return __builtin_bit_cast(uint16_t, h); }

// Store value of an fp32 result: round to nearest-even, then replace any NaN
// by the canonical quiet NaN 0x7E00 so the all-ones sentinel is never stored
// (sentinel guide, 4.6.4.3 Producer Rules).  Applied under every policy so
// the stored bits do not depend on the policy.
__device__ __forceinline__ uint16_t f32_to_f16_canon(float v) {
  uint16_t b = f16_bits((f16)v);
  return ((b & 0x7FFFu) > 0x7C00u) ? (uint16_t)0x7E00u : b;
}

// The same for bf16 (1 sign, 8 exponent, 7 fraction bits: the upper half of
// an fp32): round to nearest-even on the fp32 bit pattern (adding 0x7FFF plus
// the lowest kept bit carries into the kept half exactly when the dropped
// half is above one half, or equal to it with an odd kept part; overflow
// carries into the infinity pattern), and any NaN becomes the quiet NaN
// 0x7FC0, so the all-ones sentinel, itself a bf16 NaN, is never stored.
__device__ __forceinline__ uint16_t f32_to_bf16_canon(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Nonzero iff some 16-bit element of v is 0xFFFF: with y = ~v, a halfword of y
// is zero exactly when (y - 0x0001) & ~y has its top bit set in that halfword
// and no lower halfword is zero (a borrow only starts at a zero halfword, so
// the "some halfword" answer is exact).  Pure VALU, so the per-step check of
// a whole stage reduces to one compare and one branch.
__device__ __forceinline__ uint32_t sentinel_bits(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t y = ~v[i];
    m |= (y - 0x00010001u) & ~y & 0x80008000u;
  }
  return m;
}

__device__ __forceinline__ bool has_sentinel16(u32x4 v) {
  bool s = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s |= (v[i] & 0xFFFFu) == 0xFFFFu;
    s |= (v[i] >> 16) == 0xFFFFu;
  }
  return s;
}

// ---------------------------------------------------------------------------
// Activations on the fp32 accumulator.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float apply_act(int act, float x) {
  switch (act) {
    case kGeluErf:
      return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
    case kGeluTanh: {
      const float c = 0.79788456080286535588f;  // sqrt(2/pi)
      return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
    }
    case kRelu:
      return x < 0.0f ? 0.0f : x;
    default:
      return x;
  }
}

// Index of the XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ int xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
  return (int)(v & (kNumQueues - 1));
}

// Realtime counter for the optional per-item trace (TraceRec).
__device__ __forceinline__ uint64_t now_rt() { return __builtin_amdgcn_s_memrealtime(); }

// Where this wave runs: HW_ID gives CU [11:8], SH [12], SE [15:13].
__device__ __forceinline__ uint16_t hw_location() {
  uint32_t hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  const uint32_t cu = (hw >> 8) & 15u, sh = (hw >> 12) & 1u, se = (hw >> 13) & 7u;
  return (uint16_t)(((uint32_t)xcc_id() << 8) | (se << 5) | (sh << 4) | cu);
}

// Small deterministic per-tile hash for the delay-injection test knob.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ void debug_delay(uint32_t item, uint32_t delay) {
  if (delay == 0) return;
  const uint32_t n = (mix32(item) & 7u) * delay;
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(63);
}

}  // namespace tls
