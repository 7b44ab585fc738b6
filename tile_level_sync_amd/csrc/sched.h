// Persistent work scheduler shared by the chain kernels.
//
// Work items [0, P) are producer tiles and [P, P + C) consumer tiles.  Two
// schemes (cuSync paper, sections "Stage Processing Order" and "Tile
// Processing Order"; the paper's wait-kernel exists to give producers
// priority, which the item order gives here):
//   global  one atomic counter over [t_begin, t_end), optionally through an
//           order table that lists every consumer after the producers it reads;
//   queues  one queue per XCD per phase (0 producers, 1 consumers).  Queue q
//           holds a slab of the tile grid (columns for the MLP: each weight
//           panel is read by one XCD; or rows, which keep a conv pixel tile
//           and its halo neighbours on one XCD, but measured slower than the
//           global counter there).  A workgroup drains its
//           home queue, then the others, phase by phase, so it takes a
//           consumer only after every producer queue was found exhausted.
// Either way a consumer only waits on producer tiles already taken by running
// workgroups and producers never wait: the chain cannot deadlock, whatever
// number of workgroups is resident.
#pragma once

#include "device.h"

namespace tls {

// Item i of queue q in phase ph when no table is given: the queue's slab of
// the phase's tile grid, row by row (or column by column).
__device__ __forceinline__ uint32_t slab_item(const SchedParams& s, int ph, int q, uint32_t i) {
  const uint32_t nt = (uint32_t)s.cols[ph], nr = (uint32_t)s.rows[ph];
  uint32_t r, c;
  if (s.slab_rows) {
    const uint32_t r0 = slab_begin(q, nr), n = slab_begin(q + 1, nr) - r0;
    if (s.col_major[ph]) {
      c = i / n;
      r = r0 + i % n;
    } else {
      r = r0 + i / nt;
      c = i % nt;
    }
  } else {
    const uint32_t c0 = slab_begin(q, nt), nc = slab_begin(q + 1, nt) - c0;
    if (s.col_major[ph]) {
      c = c0 + i / nr;
      r = i % nr;
    } else {
      r = i / nc;
      c = c0 + i % nc;
    }
  }
  return s.base[ph] + r * nt + c;
}

// Next work item (thread 0 only); kNoItem when this workgroup is done.
struct SchedState {
  int phase, qo, home;
  __device__ __forceinline__ void init(const SchedParams& s) {
    phase = s.first_phase;
    qo = 0;
    home = xcc_id();
  }
  __device__ __forceinline__ uint32_t next(const SchedParams& s) {
    if (ld_relaxed_agent(&s.ctl->abort)) return kNoItem;
    if (!s.sched) {
      const uint32_t t = s.t_begin + add_relaxed_agent(&s.ctl->work, 1u);
      if (t >= s.t_end) return kNoItem;
      return s.order ? s.order[t] : t;
    }
    while (phase <= s.last_phase) {
      const int q = (home + qo) & (kNumQueues - 1);
      const uint32_t cnt = s.qcount[phase][q];
      if (cnt) {
        const uint32_t i = add_relaxed_agent(&s.ctl->qnext[phase * kNumQueues + q][0], 1u);
        if (i < cnt) return s.order ? s.order[s.qstart[phase][q] + i] : slab_item(s, phase, q, i);
      }
      if (++qo == kNumQueues) {
        qo = 0;
        ++phase;
      }
    }
    return kNoItem;
  }
};

// First items (global scheme, FirstItems): a launch's first producer items
// go out through the eight per-XCD counters instead of the shared one, on
// which a launch's first claims serialise at about 13 ns each (the 768
// workgroups of the 32 x 56 x 56 x 64 conv pair took 9 us to start).  The
// workgroup that draws shared value sweep_at (the first consumer item, or the
// end of a producer-only launch) first runs whatever those counters still
// hold, so a workgroup that is never scheduled strands nothing: every
// producer item is then claimed by a running workgroup, producers never wait,
// and a consumer only waits on producer items claimed before it was drawn.
__device__ __forceinline__ uint32_t first_item_of(const FirstItems& f, uint32_t x, uint32_t i) {
  const uint32_t n = f.n > x ? (f.n - x + kNumQueues - 1) / kNumQueues : 0u;
  return i < n ? f.base + x + i * (uint32_t)kNumQueues : kNoItem;
}

// The next item (thread 0).  `first`: the workgroup's first claim.  *sweep is
// set when the caller must run sweep_first before the returned item.
__device__ __forceinline__ uint32_t next_item(SchedState& st, const SchedParams& s,
                                              const FirstItems& f, bool first, int* sweep) {
  *sweep = 0;
  if (f.n == 0) return st.next(s);
  if (first && !(f.skip && (blockIdx.x & 1u))) {
    const uint32_t x = (uint32_t)xcc_id();
    if (f.n > x) {
      const uint32_t it = first_item_of(f, x, add_relaxed_agent(&s.ctl->qnext[x][0], 1u));
      if (it != kNoItem) return it;
    }
  }
  // the shared counter, from after the first items (no order table with them)
  const uint32_t t = s.t_begin + add_relaxed_agent(&s.ctl->work, 1u);
  *sweep = t == f.sweep_at ? 1 : 0;
  return (ld_relaxed_agent(&s.ctl->abort) || t >= s.t_end) ? kNoItem : t;
}

// Run every item the per-XCD first-item counters still hold (all threads);
// run(item) processes one producer item with the whole workgroup.  Lanes 0-7
// probe the eight counters in parallel, again while a probe found an item.
template <class RUN>
__device__ __forceinline__ void sweep_first(const FirstItems& f, Ctl* ctl, uint32_t* s_items,
                                            int* s_any, RUN&& run) {
  for (;;) {
    if (threadIdx.x < kNumQueues) {
      const uint32_t x = threadIdx.x;
      s_items[x] =
          f.n > x ? first_item_of(f, x, add_relaxed_agent(&ctl->qnext[x][0], 1u)) : kNoItem;
    }
    __syncthreads();
    bool any = false;
    for (int x = 0; x < kNumQueues; ++x) {
      const uint32_t item = s_items[x];
      if (item == kNoItem) continue;
      any = true;
      run(item);
    }
    if (threadIdx.x == 0) *s_any = any ? 1 : 0;
    __syncthreads();  // s_items and s_any read by everyone before they change
    const int again = *s_any;
    __syncthreads();
    if (!again) break;
  }
}

// Sentinel buffer rotation (sentinel guide, 4.6.4.5 Buffer Reuse): while
// this call consumes one slot of a ring of intermediate buffers, the slot the
// next call will consume is set back to the sentinel.  Nothing in this launch
// reads or writes that slot, and stream order puts the fill before the next
// call's producers.  Every workgroup claims 128 KiB chunks as it leaves the
// work loop, so the workgroups that run out of tiles first do most of it, and
// the slot is complete even when a wait expired (an incomplete slot could
// hand stale values to the next call).  All threads of the workgroup call it.
constexpr uint32_t kFillChunk = 128u * 1024u;
__device__ __forceinline__ void sentinel_refill(Ctl* ctl, void* dst, uint32_t bytes,
                                                uint32_t* s_i) {
  if (bytes == 0u) return;
  const uint32_t n = (bytes + kFillChunk - 1u) / kFillChunk;
  const auto rs = make_rsrc(dst, bytes);  // stores past the slot are dropped
  const u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  for (;;) {
    if (threadIdx.x == 0) *s_i = add_relaxed_agent(&ctl->fillnext, 1u);
    __syncthreads();
    const uint32_t i = *s_i;
    __syncthreads();  // everyone has read s_i before thread 0 claims again
    if (i >= n) break;
    for (uint32_t off = threadIdx.x * 16u; off < kFillChunk; off += blockDim.x * 16u)
      publish16(rs, i * kFillChunk + off, v);
  }
}

// Exit protocol: the last workgroup out resets the counters (and the RowSync
// counters of this launch) so the next launch starts from zero without a
// memset, and publishes the epoch of a TileSync-style call.  All threads of
// the workgroup call it.
__device__ __forceinline__ void sched_finish(const SchedParams& s, int* s_last, bool rowsync,
                                             uint32_t* rowcnt, int nrowcnt, bool tileflags,
                                             uint32_t epoch, uint32_t* splitcnt = nullptr,
                                             int nsplitcnt = 0) {
  if (threadIdx.x == 0) {
    const uint32_t d = add_relaxed_agent(&s.ctl->done, 1u);
    *s_last = (d == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (*s_last) {
    fence_acquire_agent();
    if (rowsync)
      for (int r = threadIdx.x; r < nrowcnt; r += blockDim.x) rowcnt[r * kFlagStride] = 0u;
    for (int r = threadIdx.x; r < nsplitcnt; r += blockDim.x) splitcnt[r * kFlagStride] = 0u;
    if (threadIdx.x < kMaxPhases * kNumQueues) s.ctl->qnext[threadIdx.x][0] = 0u;
    if (threadIdx.x == 0) {
      s.ctl->work = 0u;
      s.ctl->done = 0u;
      s.ctl->abort = 0u;
      s.ctl->fillnext = 0u;
      if (tileflags) s.ctl->epoch = epoch;
    }
  }
}

}  // namespace tls
